// fp32 im2win convolution on the vector ALUs.
//
// The full-precision half of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract: full
// precision on the general-purpose cores), written for CDNA4 wave64:
//
//  * Output pixels are numbered over the whole batch, q = (n*Ho + ho)*Wo + wo.
//    A workgroup owns P = 64*PX consecutive pixels and up to 128 output
//    channels (one wave per 8 channels). Lane l of a wave owns pixels
//    q0 + l + 64*j, j < PX, so only the last tile of the launch has idle
//    lanes, and the staged rows are shared by every output channel.
//  * Per stage the workgroup holds, for CIC input channels, the im2win rows
//    of every output row its pixels touch: LDS row (cc, r) for output row
//    (n, ho) holds input rows ho*sh .. ho*sh+Hf-1 column by column, so the
//    window of output column wo is the contiguous run starting at wo*sw*Hf
//    (the transform of "Im2win: Memory Efficient Convolution On SIMD
//    Architectures", Abstract). Fused launches build these rows from x (each
//    thread owns an input column and walks its Hf taps); materialised
//    launches copy them contiguously from the packed tensor. In LDS each row
//    is kept phase-major (columns grouped by col mod sw), which keeps every
//    stride-phase run of a window contiguous and puts neighbouring output
//    columns an odd number of words apart.
//  * For each window element a lane reads one LDS value per pixel and
//    multiplies it by 8 filter taps that are the same for the whole wave.
//    The taps are scalar loads into SGPRs, a few window columns at a time
//    (scheduling barriers keep the compiler from hoisting them all, which
//    would spill SGPRs), so every LDS read feeds 8 fused multiply-adds.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace im2win {

namespace {

constexpr int kMaxThreads = 1024;

struct F32Args {
    ConvShape c;
    int co_tile;               // output channels per workgroup (8 per wave)
    int P;                     // pixels per workgroup (64 * PX)
    int px_tiles, co_tiles;
    int rows_max;              // output rows one tile can touch
    int CIC;                   // input channels per LDS stage
    int NU, HFP;               // columns per stride phase ceil(Wi/sw); Hf rounded up to odd
    int RS, CS;                // LDS floats per (channel, row) and per channel
    int tpr_shift;             // log2(threads per staged segment)
    int L;                     // im2win row length Wi*Hf
    int64_t total;             // N*Ho*Wo pixels in this launch
    FastDiv divWo, divHo, divHf, divS, divRows;
};

// LDS position of im2win element (col, kh) inside one staged row. The row is
// stored phase-major: the columns of column-stride phase p = col % sw come
// first as one run (col / sw ascending), each column's Hf taps contiguous
// (HFP apart).
// Consecutive output columns then sit HFP (odd) floats apart, so the 64
// lanes of a wave read distinct LDS banks.
template <int S>
__device__ __forceinline__ int lds_pos_t(int col, int kh, int s, const F32Args& a)
{
    const int u = S ? col / S : (int)a.divS.div((uint32_t)col);
    return ((col - u * s) * a.NU + u) * a.HFP + kh;
}
#define lds_pos(col, kh, s, a) lds_pos_t<S>(col, kh, s, a)

template <int HF, int WF, int S, int PX, int COW, bool FROM_WS>
__global__ __launch_bounds__(kMaxThreads) void conv_f32_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ ws,
                                                            const float* __restrict__ w,
                                                            float* __restrict__ y, F32Args a)
{
    extern __shared__ __align__(16) float lds[];
    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co;
    const int Ho = a.c.Ho, Wo = a.c.Wo;
    const int Hf = HF ? HF : a.c.Hf;
    const int Wf = WF ? WF : a.c.Wf;
    const int sw = S ? S : a.c.sw;    // S: the column stride when fixed
    const int HW = Hf * Wf;
    const int K = Ci * HW;
    // Window columns per batch of scalar tap loads: COW*KWC SGPRs per batch.
    constexpr int KWC0 = COW <= 8 ? 4 : (COW <= 12 ? 4 : 3);
    constexpr int KWC = WF == 0 ? 1 : (WF > KWC0 + 2 ? KWC0 : WF);
    constexpr int kCoPerWave = COW;
    constexpr int NPH = S == 0 ? 1 : S;                   // phases with their own base
    constexpr int HFPC = HF | 1;                          // HFP when HF is fixed

    const int co_t = blockIdx.x % a.co_tiles;
    const int64_t q0 = (int64_t)(blockIdx.x / a.co_tiles) * a.P;
    const int64_t qend = q0 + a.P < a.total ? q0 + a.P : a.total;
    const int row0 = (int)(q0 / Wo);
    const int nrows = (int)((qend - 1) / Wo) - row0 + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int co_w = co_t * a.co_tile + wave * kCoPerWave;

    // Pixel slots of this lane and their LDS bases, one per stride phase.
    int pbase[PX][NPH], prow[PX], pwo[PX];
    bool pok[PX];
#pragma unroll
    for (int j = 0; j < PX; ++j) {
        const int64_t q = q0 + lane + 64 * j;
        pok[j] = q < qend;
        const int qq = (int)((pok[j] ? q : q0) - (int64_t)row0 * Wo);
        const int r = (int)a.divWo.div((uint32_t)qq);
        const int wo = qq - r * Wo;
        prow[j] = row0 + r;
        pwo[j] = wo;
#pragma unroll
        for (int p = 0; p < NPH; ++p) pbase[j][p] = r * a.RS + (p * a.NU + wo) * a.HFP;
    }

    // Filter rows of this wave's channels (clamped; clamped ones are not stored).
    const float* wrow[kCoPerWave];
#pragma unroll
    for (int i = 0; i < kCoPerWave; ++i) wrow[i] = w + (int64_t)min(co_w + i, Co - 1) * K;

    float acc[kCoPerWave][PX];
#pragma unroll
    for (int i = 0; i < kCoPerWave; ++i)
#pragma unroll
        for (int j = 0; j < PX; ++j) acc[i][j] = 0.f;

    const int nthr = blockDim.x;
    const int tpr = 1 << a.tpr_shift;
    const int gsub = tid >> a.tpr_shift, csub = tid & (tpr - 1);
    const int gstep = nthr >> a.tpr_shift;

    for (int c0 = 0; c0 < Ci; c0 += a.CIC) {
        const int ncs = min(a.CIC, Ci - c0);
        __syncthreads();
        // Segments (cc, r): one im2win row each. Thread groups of tpr take
        // segments in turn; segment index = cc*rows_max + r.
        for (int sg = gsub < gstep ? gsub : ncs * a.rows_max; sg < ncs * a.rows_max; sg += gstep) {
            const int cc = (int)a.divRows.div((uint32_t)sg), r = sg - cc * a.rows_max;
            if (r >= nrows) continue;
            const int gr = row0 + r;
            const int n = (int)a.divHo.div((uint32_t)gr), ho = gr - n * Ho;
            float* l = lds + cc * a.CS + r * a.RS;
            if (!FROM_WS) {
                // im2win element (col, kh) = x[n][c0+cc][ho*sh + kh][col]: the
                // Hf input rows are consecutive in x.
                const float* g = x + (((int64_t)n * Ci + c0 + cc) * Hi + ho * a.c.sh) * Wi;
                for (int col = csub; col < Wi; col += tpr) {
                    float* ld = l + lds_pos(col, 0, sw, a);
#pragma unroll 4
                    for (int kh = 0; kh < Hf; ++kh) ld[kh] = g[kh * Wi + col];
                }
            } else {
                // Row (n, c0+cc, ho) of the packed tensor, element e = col*Hf + kh.
                const float* g = ws + (((int64_t)n * Ci + c0 + cc) * Ho + ho) * a.L;
                for (int e = csub; e < a.L; e += tpr) {
                    const int col = HF ? e / HF : (int)a.divHf.div((uint32_t)e);
                    l[lds_pos(col, e - col * Hf, sw, a)] = g[e];
                }
            }
        }
        __syncthreads();

        for (int cc = 0; cc < ncs; ++cc) {
            const int wofs = (c0 + cc) * HW;
#pragma unroll 1
            for (int kh = 0; kh < Hf; ++kh) {
                const int wk = wofs + kh * Wf;
                if (WF != 0 && S != 0) {
                    int base[PX][NPH];
#pragma unroll
                    for (int j = 0; j < PX; ++j)
#pragma unroll
                        for (int p = 0; p < NPH; ++p) base[j][p] = cc * a.CS + pbase[j][p] + kh;
#pragma unroll
                    for (int kw0 = 0; kw0 < WF; kw0 += KWC) {
                        float wv[kCoPerWave][KWC];
#pragma unroll
                        for (int i = 0; i < kCoPerWave; ++i)
#pragma unroll
                            for (int q = 0; q < KWC; ++q)
                                wv[i][q] = kw0 + q < WF ? wrow[i][wk + kw0 + q] : 0.f;
#pragma unroll
                        for (int q = 0; q < KWC; ++q) {
                            const int kw = kw0 + q;
                            if (kw >= WF) break;
                            float xv[PX];
#pragma unroll
                            for (int j = 0; j < PX; ++j)
                                xv[j] = lds[base[j][kw % NPH] + (kw / NPH) * HFPC];
#pragma unroll
                            for (int i = 0; i < kCoPerWave; ++i)
#pragma unroll
                                for (int j = 0; j < PX; ++j)
                                    acc[i][j] = __builtin_fmaf(xv[j], wv[i][q], acc[i][j]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
                    for (int kw = 0; kw < Wf; ++kw) {
                        const int ph = kw % sw, adv = kw / sw;
                        float xv[PX];
#pragma unroll
                        for (int j = 0; j < PX; ++j)
                            xv[j] = lds[cc * a.CS + pbase[j][0] + (ph * a.NU + adv) * a.HFP + kh];
#pragma unroll
                        for (int i = 0; i < kCoPerWave; ++i) {
                            const float wv = wrow[i][wk + kw];
#pragma unroll
                            for (int j = 0; j < PX; ++j)
                                acc[i][j] = __builtin_fmaf(xv[j], wv, acc[i][j]);
                        }
                    }
                }
            }
        }
    }

#pragma unroll
    for (int j = 0; j < PX; ++j) {
        if (!pok[j]) continue;
        const int n = (int)a.divHo.div((uint32_t)prow[j]), ho = prow[j] - n * Ho;
        float* yp = y + (((int64_t)n * Co + co_w) * Ho + ho) * Wo + pwo[j];
#pragma unroll
        for (int i = 0; i < kCoPerWave; ++i)
            if (co_w + i < Co) yp[(int64_t)i * Ho * Wo] = acc[i][j];
    }
}

template <int HF, int WF, int S, int PX, int COW>
void launch_t(const float* x, const float* ws, const float* w, float* y, const F32Args& a,
              unsigned blocks, unsigned threads, size_t lds, hipStream_t stream)
{
    if (ws)
        hipLaunchKernelGGL((conv_f32_kernel<HF, WF, S, PX, COW, true>), dim3(blocks),
                           dim3(threads), lds, stream, x, ws, w, y, a);
    else
        hipLaunchKernelGGL((conv_f32_kernel<HF, WF, S, PX, COW, false>), dim3(blocks),
                           dim3(threads), lds, stream, x, ws, w, y, a);
}

template <int HF, int WF, int S>
void launch_px(int px, int cow, const float* x, const float* ws, const float* w, float* y,
               const F32Args& a, unsigned blocks, unsigned threads, size_t lds, hipStream_t stream)
{
#define IM2WIN_F32_CASE(P, C)                                                               \
    if (px == P && cow == C) {                                                            \
        launch_t<HF, WF, S, P, C>(x, ws, w, y, a, blocks, threads, lds, stream);          \
        return;                                                                           \
    }
    IM2WIN_F32_CASE(4, 8) IM2WIN_F32_CASE(2, 8) IM2WIN_F32_CASE(1, 8)
#undef IM2WIN_F32_CASE
}

int log2_ceil_pow2(int v, int cap)
{
    int sh = 0;
    while ((1 << sh) < v && (2 << sh) <= cap) ++sh;
    return sh;
}

}  // namespace

// Tuning overrides for experiments (0 = choose automatically).
#ifndef IM2WIN_F32_PX
#define IM2WIN_F32_PX 0
#endif
#ifndef IM2WIN_F32_WAVES
#define IM2WIN_F32_WAVES 0
#endif

int launch_conv_f32(const float* x, const float* ws, const float* w, float* y,
                    const ConvShape& c, hipStream_t stream)
{
    constexpr int kLdsCap = 64 * 1024;   // per workgroup
    constexpr int kCUs = 256;
    F32Args a;
    a.c = c;
    a.total = (int64_t)c.N * c.Ho * c.Wo;
    a.L = c.Wi * c.Hf;
    a.NU = ceil_div(c.Wi, c.sw);
    a.HFP = c.Hf | 1;
    a.RS = (c.sw * a.NU * a.HFP) | 1;
    if ((int64_t)c.N * c.Ho > 0x7fffffff) return -1;

    // Eight output channels per wave (wider waves spill SGPRs), up to 16
    // waves (128 channels) per workgroup so the staged rows serve as many
    // channels as possible.
    const int cow = 8;
    int waves = IM2WIN_F32_WAVES ? IM2WIN_F32_WAVES : std::min(16, ceil_div(c.Co, cow));
    a.co_tile = waves * cow;
    a.co_tiles = ceil_div(c.Co, a.co_tile);

    // Pixels per lane: the largest of 4, 2, 1 whose staged rows fit LDS and
    // that still gives every CU two workgroups; 1 otherwise.
    int best_px = 0;
    for (int px = 4; px >= 1; px /= 2) {
        if (IM2WIN_F32_PX && px != IM2WIN_F32_PX) continue;
        const int P = 64 * px;
        const int rows_max = (P - 1) / c.Wo + 2;
        if ((int64_t)rows_max * a.RS * 4 > kLdsCap) continue;
        const int64_t tiles = ((a.total + P - 1) / P) * a.co_tiles;
        best_px = px;
        if (tiles >= 2 * kCUs) break;
    }
    if (best_px == 0) return -1;   // not even one row set of a 64-pixel tile fits LDS
    const int px = best_px;
    a.P = 64 * px;
    a.rows_max = (a.P - 1) / c.Wo + 2;
    a.CS = a.rows_max * a.RS;
    a.CIC = std::max(1, std::min(c.Ci, (kLdsCap / 2) / (a.CS * 4)));
    const int threads = 64 * waves;
    a.tpr_shift = log2_ceil_pow2(ws ? a.L : c.Wi, threads);
    if ((threads >> a.tpr_shift) < 1) return -1;  // staging needs >= 1 thread group
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divHo = FastDiv((uint32_t)c.Ho);
    a.divHf = FastDiv((uint32_t)c.Hf);
    a.divS = FastDiv((uint32_t)c.sw);
    a.divRows = FastDiv((uint32_t)a.rows_max);
    a.px_tiles = (int)((a.total + a.P - 1) / a.P);
    const int64_t blocks = (int64_t)a.px_tiles * a.co_tiles;
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    const size_t lds = (size_t)a.CIC * a.CS * sizeof(float);
    const unsigned nb = (unsigned)blocks, nt = (unsigned)threads;
    // Specialised on the filter and the column stride; the row stride is a
    // run-time value in every variant.
    if (c.Hf == 11 && c.Wf == 11 && c.sw == 4) launch_px<11, 11, 4>(px, cow, x, ws, w, y, a, nb, nt, lds, stream);
    else if (c.Hf == 7 && c.Wf == 7 && c.sw == 2) launch_px<7, 7, 2>(px, cow, x, ws, w, y, a, nb, nt, lds, stream);
    else if (c.Hf == 5 && c.Wf == 5 && c.sw == 1) launch_px<5, 5, 1>(px, cow, x, ws, w, y, a, nb, nt, lds, stream);
    else if (c.Hf == 3 && c.Wf == 3 && c.sw == 1) launch_px<3, 3, 1>(px, cow, x, ws, w, y, a, nb, nt, lds, stream);
    else launch_px<0, 0, 0>(px, cow, x, ws, w, y, a, nb, nt, lds, stream);
    return launch_status();
}

}  // namespace im2win
