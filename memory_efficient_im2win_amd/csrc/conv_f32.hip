// fp32 im2win convolution on the vector ALUs.
//
// The full-precision half of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract: full
// precision on the general-purpose cores), written for CDNA4 wave64:
//
//  * Output pixels are numbered over the whole batch, q = (n*Ho + ho)*Wo + wo.
//    A workgroup owns P = 64*PX consecutive pixels and 32 output channels
//    (4 waves x 8 channels). Lane l of a wave owns pixels q0 + l + 64*j,
//    j < PX, so only the last tile of the launch has idle lanes.
//  * Per stage the workgroup holds, for CIC input channels, the im2win rows
//    of every output row its pixels touch: LDS row (cc, r) for output row
//    (n, ho) holds input rows ho*s .. ho*s+Hf-1 column by column, so the
//    window of output column wo is the contiguous run starting at wo*s*Hf
//    (the transform of "Im2win: Memory Efficient Convolution On SIMD
//    Architectures", Abstract). Fused launches build these rows from x;
//    materialised launches copy them contiguously from the packed tensor.
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

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kCoPerWave = 8;
constexpr int kCoTile = kWaves * kCoPerWave;

struct F32Args {
    ConvShape c;
    int P;                     // pixels per workgroup (64 * PX)
    int px_tiles, co_tiles;
    int rows_max;              // output rows one tile can touch
    int CIC;                   // input channels per LDS stage
    int RS, CS;                // LDS floats per (channel, row) and per channel
    int tpr_shift;             // log2(threads per staged segment)
    int L;                     // im2win row length Wi*Hf
    int64_t total;             // N*Ho*Wo pixels in this launch
    FastDiv divWo, divHo, divHf;
};

template <int HF, int WF, int PX, bool FROM_WS>
__global__ __launch_bounds__(kThreads) void conv_f32_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ ws,
                                                            const float* __restrict__ w,
                                                            float* __restrict__ y, F32Args a)
{
    extern __shared__ __align__(16) float lds[];
    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co, s = a.c.s;
    const int Ho = a.c.Ho, Wo = a.c.Wo;
    const int Hf = HF ? HF : a.c.Hf;
    const int Wf = WF ? WF : a.c.Wf;
    const int HW = Hf * Wf;
    const int K = Ci * HW;
    constexpr int KWC = WF == 0 ? 1 : (WF > 6 ? 4 : WF);  // window columns per tap batch

    const int co_t = blockIdx.x % a.co_tiles;
    const int64_t q0 = (int64_t)(blockIdx.x / a.co_tiles) * a.P;
    const int64_t qend = q0 + a.P < a.total ? q0 + a.P : a.total;
    const int row0 = (int)(q0 / Wo);
    const int nrows = (int)((qend - 1) / Wo) - row0 + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int co_w = co_t * kCoTile + wave * kCoPerWave;

    // Pixel slots of this lane.
    int pix[PX], prow[PX], pwo[PX];
    bool pok[PX];
#pragma unroll
    for (int j = 0; j < PX; ++j) {
        const int64_t q = q0 + lane + 64 * j;
        pok[j] = q < qend;
        const int qq = (int)((pok[j] ? q : q0) - (int64_t)row0 * Wo);  // offset from row0 start
        const int r = (int)a.divWo.div((uint32_t)qq);
        const int wo = qq - r * Wo;
        prow[j] = row0 + r;
        pwo[j] = wo;
        pix[j] = r * a.RS + wo * s * Hf;
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

    const int tpr = 1 << a.tpr_shift;
    const int rsub = tid >> a.tpr_shift, csub = tid & (tpr - 1);
    const int rstep = kThreads >> a.tpr_shift;

    for (int c0 = 0; c0 < Ci; c0 += a.CIC) {
        const int ncs = min(a.CIC, Ci - c0);
        __syncthreads();
        if (!FROM_WS) {
            // LDS[cc][r][col*Hf + kh] = x[n][c0+cc][ho*s + kh][col], (n, ho) = row0 + r
            const int nseg = ncs * nrows * Hf;
            for (int t = rsub; t < nseg; t += rstep) {
                const int seg = (int)a.divHf.div((uint32_t)t);  // t = seg*Hf + kh
                const int kh = t - seg * Hf;
                const int cc = seg / nrows, r = seg - cc * nrows;  // seg = cc*nrows + r
                const int gr = row0 + r;
                const int n = (int)a.divHo.div((uint32_t)gr), ho = gr - n * Ho;
                const float* g = x + (((int64_t)n * Ci + c0 + cc) * Hi + ho * s + kh) * Wi;
                float* l = lds + cc * a.CS + r * a.RS + kh;
                for (int col = csub; col < Wi; col += tpr) l[col * Hf] = g[col];
            }
        } else {
            // LDS[cc][r][e] = ws[n][c0+cc][ho][e]
            const int nseg = ncs * nrows;
            for (int t = rsub; t < nseg; t += rstep) {
                const int cc = t / nrows, r = t - (t / nrows) * nrows;
                const int gr = row0 + r;
                const int n = (int)a.divHo.div((uint32_t)gr), ho = gr - n * Ho;
                const float* g = ws + (((int64_t)n * Ci + c0 + cc) * Ho + ho) * a.L;
                float* l = lds + cc * a.CS + r * a.RS;
                for (int e = csub; e < a.L; e += tpr) l[e] = g[e];
            }
        }
        __syncthreads();

        for (int cc = 0; cc < ncs; ++cc) {
            const int wofs = (c0 + cc) * HW;
#pragma unroll 1
            for (int kh = 0; kh < Hf; ++kh) {
                int base[PX];
#pragma unroll
                for (int j = 0; j < PX; ++j) base[j] = cc * a.CS + pix[j] + kh;
                const int wk = wofs + kh * Wf;
                if (WF != 0) {
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
                            if (kw0 + q >= WF) break;
                            float xv[PX];
#pragma unroll
                            for (int j = 0; j < PX; ++j) xv[j] = lds[base[j] + (kw0 + q) * Hf];
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
                        float xv[PX];
#pragma unroll
                        for (int j = 0; j < PX; ++j) xv[j] = lds[base[j] + kw * Hf];
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

template <int HF, int WF, int PX>
void launch_t(const float* x, const float* ws, const float* w, float* y, const F32Args& a,
              unsigned blocks, size_t lds, hipStream_t stream)
{
    if (ws)
        hipLaunchKernelGGL((conv_f32_kernel<HF, WF, PX, true>), dim3(blocks), dim3(kThreads),
                           lds, stream, x, ws, w, y, a);
    else
        hipLaunchKernelGGL((conv_f32_kernel<HF, WF, PX, false>), dim3(blocks), dim3(kThreads),
                           lds, stream, x, ws, w, y, a);
}

template <int HF, int WF>
void launch_px(int px, const float* x, const float* ws, const float* w, float* y,
               const F32Args& a, unsigned blocks, size_t lds, hipStream_t stream)
{
    if (px == 4) launch_t<HF, WF, 4>(x, ws, w, y, a, blocks, lds, stream);
    else if (px == 2) launch_t<HF, WF, 2>(x, ws, w, y, a, blocks, lds, stream);
    else launch_t<HF, WF, 1>(x, ws, w, y, a, blocks, lds, stream);
}

int log2_ceil_pow2(int v, int cap)
{
    int sh = 0;
    while ((1 << sh) < v && (1 << sh) < cap) ++sh;
    return sh;
}

}  // namespace

int launch_conv_f32(const float* x, const float* ws, const float* w, float* y,
                    const ConvShape& c, hipStream_t stream)
{
    constexpr int kLdsCap = 64 * 1024;
    F32Args a;
    a.c = c;
    a.total = (int64_t)c.N * c.Ho * c.Wo;
    a.co_tiles = ceil_div(c.Co, kCoTile);
    a.L = c.Wi * c.Hf;
    a.RS = a.L | 1;
    // Pixels per lane: as many as keep >= ~2 workgroups per CU on 256 CUs.
    int px = 4;
    while (px > 1 && ceil_div((int)std::min<int64_t>(a.total, 1 << 30), 64 * px) * a.co_tiles < 512)
        px /= 2;
    // The rows one tile touches must fit LDS for at least one channel.
    for (;;) {
        a.P = 64 * px;
        a.rows_max = (a.P - 1) / c.Wo + 2;
        if ((int64_t)a.rows_max * a.RS * 4 <= kLdsCap || px == 1) break;
        px /= 2;
    }
    a.CS = a.rows_max * a.RS;
    if ((int64_t)a.CS * 4 > kLdsCap) return -1;
    a.CIC = std::max(1, std::min(c.Ci, (kLdsCap / 2) / (a.CS * 4)));
    if (a.CIC == 0) a.CIC = 1;
    a.tpr_shift = log2_ceil_pow2(ws ? a.L : c.Wi, kThreads);
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divHo = FastDiv((uint32_t)c.Ho);
    a.divHf = FastDiv((uint32_t)c.Hf);
    if ((int64_t)c.N * c.Ho > 0x7fffffff) return -1;
    a.px_tiles = (int)((a.total + a.P - 1) / a.P);
    const int64_t blocks = (int64_t)a.px_tiles * a.co_tiles;
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    const size_t lds = (size_t)a.CIC * a.CS * sizeof(float);
    const unsigned nb = (unsigned)blocks;
    if (c.Hf == 11 && c.Wf == 11) launch_px<11, 11>(px, x, ws, w, y, a, nb, lds, stream);
    else if (c.Hf == 7 && c.Wf == 7) launch_px<7, 7>(px, x, ws, w, y, a, nb, lds, stream);
    else if (c.Hf == 5 && c.Wf == 5) launch_px<5, 5>(px, x, ws, w, y, a, nb, lds, stream);
    else if (c.Hf == 3 && c.Wf == 3) launch_px<3, 3>(px, x, ws, w, y, a, nb, lds, stream);
    else launch_px<0, 0>(px, x, ws, w, y, a, nb, lds, stream);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace im2win
