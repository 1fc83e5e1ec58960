// Fused fp16 im2win convolution on the CDNA4 matrix cores (fp32 accumulate).
//
// The half-precision path of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract: half
// precision multiply-accumulate on matrix hardware) for one MI355X. The
// contraction over Ci*Hf*Wf runs on v_mfma_f32_32x32x16_f16:
//
//  * GEMM view: rows = output channels (A = filters), columns = output
//    pixels (B = windows), K = (channel group g of 8, window tap j, channel
//    in the group). Pixels are numbered over the whole batch,
//    q = (n*Ho + ho)*Wo + wo. A workgroup of WCO x WPX waves owns
//    64*WCO channels and P = 32*NB*WPX consecutive pixels; each wave owns a
//    64-channel x 32*NB-pixel block (2 x NB MFMA tiles, AGPR accumulators).
//  * Per channel group the workgroup stages in LDS the window tile of its
//    pixels: the Hf input rows of each im2win row it needs, channel-
//    interleaved (16-byte entry = 8 channels of one input pixel), each input
//    row stored once even where the im2win rows of consecutive output rows
//    overlap (s < Hf). Output rows of different images get separate rows.
//    The window of a pixel is then Hf runs of Wf entries, and every lane's
//    8-element K slice of B is one 16-byte LDS read.
//  * The filters of the group are staged as entries (tap j, channel co) in
//    the same K order, from the caller's prepacked copy when a workspace is
//    given (contiguous 16-byte loads) or gathered from w otherwise.
//  * The next group's global loads are issued into registers before the
//    MFMAs of the current group and written to LDS after them, so HBM/L2
//    latency overlaps the matrix work.
//  * One MFMA consumes two taps (j = 2t for lanes 0-31, 2t+1 for 32-63); an
//    odd tap count gets a zero filter entry and a zeroed B slice, so an
//    infinity next to a window never turns into NaN.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace im2win {

namespace {

constexpr int kMaxLds = 160 * 1024;
constexpr int kCoPad = 128;   // prepacked filter: channels padded to a multiple of this

struct FusedArgs {
    ConvShape c;
    int P, co_tile, co_tiles;
    int64_t px_tiles, total;
    int rows_max, kmax, dup, RIN;   // output rows per tile, image breaks, s<Hf overlap, LDS rows
    int HW, HWp, CG, Copad;
    int xentries;                   // RIN * Wi
    int xunits;                     // RIN * Wi / 8 (vector staging)
    bool xvec;                      // Wi % 8 == 0: rows fetched as 16-byte vectors
    FastDiv divWo, divHo, divWi, divHWp, divCot;
};

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi)
{
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Filters of channel group g as 16-byte entries (tap j, channel co):
// wpk[(g*HWp + j)*Copad + co] = w[co][8g..8g+7][j], zero beyond Co, Ci, HW.
__global__ __launch_bounds__(256) void f16_filter_pack_kernel(const uint16_t* __restrict__ w,
                                                              uint4* __restrict__ wpk,
                                                              FusedArgs a)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)a.CG * a.HWp * a.Copad;
    if (e >= total) return;
    const int co = (int)(e % a.Copad);
    const int64_t gj = e / a.Copad;
    const int j = (int)(gj % a.HWp), g = (int)(gj / a.HWp);
    uint16_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (co < a.c.Co && j < a.HW) {
        const uint16_t* src = w + ((int64_t)co * a.c.Ci + 8 * g) * a.HW + j;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (8 * g + q < a.c.Ci) v[q] = src[(int64_t)q * a.HW];
    }
    wpk[e] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]),
                        pack2(v[6], v[7]));
}

// Per-thread staging capacities (checked by the planner).
constexpr int kXUnits = 2;    // input units of 8 columns x 8 channels (vector path)
constexpr int kXEnt = 10;     // input entries (gather path)
constexpr int kWEnt = 8;      // filter entries

template <int WCO, int WPX, int NB, bool XVEC, bool WPK>
__global__ __launch_bounds__(64 * WCO * WPX) void conv_f16_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint4* __restrict__ wpk, float* __restrict__ y, FusedArgs a)
{
    constexpr int NT = 64 * WCO * WPX;
    constexpr int COT = 64 * WCO;

    extern __shared__ __align__(16) uint4 lds[];
    uint4* X = lds;
    uint4* Wl = lds + a.xentries;

    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co, s = a.c.s;
    const int Ho = a.c.Ho, Wo = a.c.Wo, Hf = a.c.Hf, Wf = a.c.Wf;
    const int HW = a.HW, HWp = a.HWp;

    const int co_t = (int)(blockIdx.x % a.co_tiles);
    const int64_t pt = blockIdx.x / a.co_tiles;
    const int co0 = co_t * COT;
    const int64_t q0 = pt * a.P;
    const int64_t qend = q0 + a.P < a.total ? q0 + a.P : a.total;
    const int gr0 = (int)(q0 / Wo);
    const int grl = (int)((qend - 1) / Wo);
    const int n0 = (int)a.divHo.div((uint32_t)gr0);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int wave = uniform(tid >> 6);
    const int wco = wave % WCO, wpx = wave / WCO;

    // LDS row of output row gr (tile-relative r = gr - gr0, image k):
    // r*s + k*dup; its kh-th input row sits kh rows further.
    int xb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        int64_t q = q0 + (wpx * NB + b) * 32 + l32;
        if (q >= qend) q = qend - 1;
        const int gr = (int)a.divWo.div((uint32_t)(q - (int64_t)gr0 * Wo)) + gr0;
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int k = (int)a.divHo.div((uint32_t)gr) - n0;
        xb[b] = ((gr - gr0) * s + k * a.dup) * Wi + wo * s;
    }
    const int arow = wco * 64 + l32;   // A entry column for co block 0 of this wave

    floatx16_t acc[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][b][r] = 0.f;

    // LDS row i -> (image n, input row h); false if no input row maps there.
    // Segment k holds the output rows of image n0+k that fall in the tile.
    auto x_src = [&](int i, int& n, int& h) -> bool {
        for (int k = 0; k <= a.kmax; ++k) {
            const int nk = n0 + k;
            const int first = max(gr0, nk * Ho), last = min(grl, nk * Ho + Ho - 1);
            if (first > last) break;
            const int S = (first - gr0) * s + k * a.dup;
            const int span = (last - first) * s + Hf;
            if (i >= S && i < S + span) {
                n = nk;
                h = (first - nk * Ho) * s + (i - S);
                return true;
            }
        }
        return false;
    };

    // ---- staging: global -> registers (group g) -> LDS --------------------------
    // Vector path: a unit is 8 consecutive columns of one LDS row; it is
    // fetched as 8 channels x 16 bytes and transposed into 8 entries.
    uint4 xv[XVEC ? kXUnits * 8 : 1];
    uint4 xg[XVEC ? 1 : kXEnt];
    uint4 wv[kWEnt];
    const int wcols = Wi >> 3;

    auto load_group = [&](int g) {
        const int cb = 8 * g;
        const int64_t cstride = (int64_t)Hi * Wi;
        if (XVEC) {
#pragma unroll
            for (int u = 0; u < kXUnits; ++u) {
                const int e = tid + u * NT;          // unit = (row i, column block)
                const int i = e / wcols, cblk = e - (e / wcols) * wcols;
                int n = 0, h = 0;
                const bool ok = e < a.xunits && x_src(i, n, h);
                const uint4* src = reinterpret_cast<const uint4*>(
                    x + (((int64_t)n * Ci + cb) * Hi + h) * Wi + cblk * 8);
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    xv[u * 8 + q] = ok && cb + q < Ci ? src[q * (cstride >> 3)] : make_uint4(0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int u = 0; u < kXEnt; ++u) {
                const int e = tid + u * NT;
                uint32_t v[4] = {0, 0, 0, 0};
                if (e < a.xentries) {
                    const int i = (int)a.divWi.div((uint32_t)e), col = e - i * Wi;
                    int n, h;
                    if (x_src(i, n, h)) {
                        const uint16_t* src = x + (((int64_t)n * Ci + cb) * Hi + h) * Wi + col;
#pragma unroll
                        for (int q = 0; q < 8; ++q)
                            if (cb + q < Ci) v[q >> 1] |= (uint32_t)src[q * cstride] << (16 * (q & 1));
                    }
                }
                xg[u] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        }
        const int wentries = HWp * COT;
#pragma unroll
        for (int u = 0; u < kWEnt; ++u) {
            const int e = tid + u * NT;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (e < wentries) {
                const int j = e / COT, col = e - (e / COT) * COT;
                if (WPK) {
                    val = wpk[((int64_t)g * HWp + j) * a.Copad + co0 + col];
                } else if (j < HW && co0 + col < Co) {
                    const uint16_t* src = w + ((int64_t)(co0 + col) * Ci + cb) * HW + j;
                    uint32_t v[4] = {0, 0, 0, 0};
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        if (cb + q < Ci) v[q >> 1] |= (uint32_t)src[q * HW] << (16 * (q & 1));
                    val = make_uint4(v[0], v[1], v[2], v[3]);
                }
            }
            wv[u] = val;
        }
    };
    auto store_group = [&]() {
        if (XVEC) {
#pragma unroll
            for (int u = 0; u < kXUnits; ++u) {
                const int e = tid + u * NT;
                if (e >= a.xunits) continue;
                const int i = e / wcols, cblk = e - (e / wcols) * wcols;
                uint4* dst = X + i * Wi + cblk * 8;
                // d[c] = columns 0..7 of channel c; entry m = channels 0..7 of column m.
                const uint32_t* d = reinterpret_cast<const uint32_t*>(&xv[u * 8]);
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int sh = 16 * (m & 1), k = m >> 1;
                    uint32_t e4[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const uint32_t lo = (d[(2 * p) * 4 + k] >> sh) & 0xffffu;
                        const uint32_t hi = (d[(2 * p + 1) * 4 + k] >> sh) & 0xffffu;
                        e4[p] = lo | (hi << 16);
                    }
                    dst[m] = make_uint4(e4[0], e4[1], e4[2], e4[3]);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < kXEnt; ++u) {
                const int e = tid + u * NT;
                if (e < a.xentries) X[e] = xg[u];
            }
        }
        const int wentries = HWp * COT;
#pragma unroll
        for (int u = 0; u < kWEnt; ++u) {
            const int e = tid + u * NT;
            if (e < wentries) Wl[e] = wv[u];
        }
    };

    const int nsteps = HWp >> 1;
    const bool odd = (HW & 1) != 0;

    load_group(0);
    store_group();
    __syncthreads();
    for (int g = 0; g < a.CG; ++g) {
        if (g + 1 < a.CG) load_group(g + 1);

        // Tap pair t: lanes 0-31 take tap 2t, lanes 32-63 tap 2t+1, taps in
        // filter order j = kh*Wf + kw.
        int kh = 0, kw = hl;
        if (kw >= Wf) { kw -= Wf; ++kh; }
        for (int t = 0; t < nsteps; ++t) {
            const bool zero_b = odd && hl && t == nsteps - 1;   // padding tap j = HW
            const int off = zero_b ? 0 : kh * Wi + kw;
            half8_t av[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 u = Wl[(2 * t + hl) * COT + arow + i * 32];
                __builtin_memcpy(&av[i], &u, 16);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                uint4 u = X[xb[b] + off];
                if (zero_b) u = make_uint4(0, 0, 0, 0);
                half8_t bv;
                __builtin_memcpy(&bv, &u, 16);
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv, acc[i][b], 0, 0, 0);
            }
            kw += 2;
            while (kw >= Wf) { kw -= Wf; ++kh; }
        }

        if (g + 1 < a.CG) {
            __syncthreads();
            store_group();
            __syncthreads();
        }
    }

    // Output: lane holds pixel l32 of each block and channels
    // 8*(r/4) + 4*hl + r%4 of each 32-channel block.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int64_t q = q0 + (wpx * NB + b) * 32 + l32;
        if (q >= qend) continue;
        const int gr = (int)(q / Wo);
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int n = (int)a.divHo.div((uint32_t)gr), ho = gr - n * Ho;
        float* yp = y + ((int64_t)n * Co * Ho + ho) * Wo + wo;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = co0 + wco * 64 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (co < Co) yp[(int64_t)co * Ho * Wo] = acc[i][b][r];
            }
    }
}

// Plans the fused launch; returns false if the shape is outside its envelope.
bool plan(const ConvShape& c, FusedArgs& a, int& wco, int& wpx, int& nb)
{
    a.c = c;
    a.HW = c.Hf * c.Wf;
    a.HWp = (a.HW + 1) & ~1;
    a.CG = ceil_div(c.Ci, 8);
    a.Copad = ceil_div(c.Co, kCoPad) * kCoPad;
    a.total = (int64_t)c.N * c.Ho * c.Wo;
    a.dup = std::max(0, c.Hf - c.s);
    if ((int64_t)c.N * c.Ho > 0x7fffffff) return false;
    nb = 2;
    wco = c.Co > 64 ? 2 : 1;
    a.xvec = c.Wi % 8 == 0;
    for (wpx = 8 / wco; wpx >= 1; wpx /= 2) {
        a.co_tile = 64 * wco;
        a.P = 32 * nb * wpx;
        a.rows_max = (a.P - 1) / c.Wo + 2;
        a.kmax = a.rows_max > 1 ? ceil_div(a.rows_max - 1, c.Ho) : 0;
        a.RIN = (a.rows_max - 1) * c.s + c.Hf + a.kmax * a.dup;
        a.xentries = a.RIN * c.Wi;
        const int nt = 64 * wco * wpx;
        const int wentries = a.HWp * a.co_tile;
        const int64_t bytes = ((int64_t)a.xentries + wentries) * 16;
        const bool xfit = a.xvec ? a.xentries / 8 <= kXUnits * nt : a.xentries <= kXEnt * nt;
        if (bytes <= kMaxLds && xfit && wentries <= kWEnt * nt) break;
    }
    if (wpx < 1) return false;
    a.xunits = a.xentries / 8;
    a.co_tiles = ceil_div(c.Co, a.co_tile);
    a.px_tiles = (a.total + a.P - 1) / a.P;
    if (a.px_tiles * a.co_tiles > 0x7fffffff) return false;
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divHo = FastDiv((uint32_t)c.Ho);
    a.divWi = FastDiv((uint32_t)c.Wi);
    a.divHWp = FastDiv((uint32_t)a.HWp);
    a.divCot = FastDiv((uint32_t)a.co_tile);
    return true;
}

template <int WCO, int WPX, int NB, bool XVEC, bool WPK>
int launch_t(const uint16_t* x, const uint16_t* w, const uint4* wpk, float* y,
             const FusedArgs& a, hipStream_t stream)
{
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute((const void*)conv_f16_fused_kernel<WCO, WPX, NB, XVEC, WPK>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        attr = true;
    }
    const size_t lds = ((size_t)a.xentries + (size_t)a.HWp * a.co_tile) * 16;
    hipLaunchKernelGGL((conv_f16_fused_kernel<WCO, WPX, NB, XVEC, WPK>),
                       dim3((unsigned)(a.px_tiles * a.co_tiles)), dim3(64 * WCO * WPX), lds,
                       stream, x, w, wpk, y, a);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <int WCO, int WPX>
int launch_w(const uint16_t* x, const uint16_t* w, const uint4* wpk, float* y,
             const FusedArgs& a, hipStream_t stream)
{
    if (a.xvec)
        return wpk ? launch_t<WCO, WPX, 2, true, true>(x, w, wpk, y, a, stream)
                   : launch_t<WCO, WPX, 2, true, false>(x, w, wpk, y, a, stream);
    return wpk ? launch_t<WCO, WPX, 2, false, true>(x, w, wpk, y, a, stream)
               : launch_t<WCO, WPX, 2, false, false>(x, w, wpk, y, a, stream);
}

}  // namespace

size_t f16_filter_pack_bytes(const ConvShape& c)
{
    FusedArgs a;
    int wco, wpx, nb;
    if (!plan(c, a, wco, wpx, nb)) return 0;
    return (size_t)a.CG * a.HWp * a.Copad * 16;
}

int launch_f16_filter_pack(const uint16_t* w, void* wpk, const ConvShape& c, hipStream_t stream)
{
    FusedArgs a;
    int wco, wpx, nb;
    if (!plan(c, a, wco, wpx, nb)) return -1;
    const int64_t total = (int64_t)a.CG * a.HWp * a.Copad;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return -1;
    hipLaunchKernelGGL(f16_filter_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w,
                       (uint4*)wpk, a);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_conv_f16_fused(const uint16_t* x, const uint16_t* w, const void* wpk, float* y,
                          const ConvShape& c, hipStream_t stream)
{
    FusedArgs a;
    int wco, wpx, nb;
    if (!plan(c, a, wco, wpx, nb)) return -1;
    const uint4* wp = static_cast<const uint4*>(wpk);
    if (wco == 1 && wpx == 8) return launch_w<1, 8>(x, w, wp, y, a, stream);
    if (wco == 1 && wpx == 4) return launch_w<1, 4>(x, w, wp, y, a, stream);
    if (wco == 1 && wpx == 2) return launch_w<1, 2>(x, w, wp, y, a, stream);
    if (wco == 1 && wpx == 1) return launch_w<1, 1>(x, w, wp, y, a, stream);
    if (wco == 2 && wpx == 4) return launch_w<2, 4>(x, w, wp, y, a, stream);
    if (wco == 2 && wpx == 2) return launch_w<2, 2>(x, w, wp, y, a, stream);
    if (wco == 2 && wpx == 1) return launch_w<2, 1>(x, w, wp, y, a, stream);
    return -1;
}

}  // namespace im2win
