// fp16 im2win convolution on the CDNA4 matrix cores (fp32 accumulate).
//
// The half-precision half of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract:
// half-precision multiply-accumulate on matrix hardware). The reduction over
// Ci*Hf*Wf is a dense contraction, so it runs on v_mfma_f32_32x32x16_f16:
//
//  * GEMM view: rows = output channels (A = filters), columns = output
//    pixels (B = windows), K = (channel group g of 8, window position j,
//    channel within the group). A workgroup owns 64 output channels (two
//    32-row blocks) and a tile of TH x TW pixels of one image (up to eight
//    32-column blocks, two per wave).
//  * LDS holds the im2win rows of the tile, channel-interleaved: entry
//    (th, col*Hf + kh) is 16 bytes = channels 8g..8g+7 of input pixel
//    ((ho0+th)*sh + kh, wo0*sw + col). Window position j = kw*Hf + kh of tile
//    pixel (th, tw) is entry th*XRS + tw*sw*Hf + j: the window is one
//    contiguous run (the transform of "Im2win: Memory Efficient Convolution
//    On SIMD Architectures", Abstract), so each lane's 8-element K slice of
//    B is one 16-byte LDS read. Fused launches build the rows from x;
//    materialised launches read them from the packed im2win tensor.
//  * The filters for group g are staged once per group into LDS in the same
//    (j, channel) order: entry (j, co) = w[co][8g..8g+7][kh][kw].
//  * One MFMA covers two window positions (j = 2t for lanes 0-31, 2t+1 for
//    lanes 32-63) x 8 channels; an odd window count is padded with a zero
//    filter entry and a zeroed B slice.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace im2win {

namespace {

constexpr int kThreads = 256;
constexpr int kCoTile = 64;
constexpr int kPxTile = 256;
constexpr int kMaxLds = 160 * 1024;

struct F16Args {
    ConvShape c;
    int TH, TW, LW, P, npb;    // tile rows/cols, staged cols, pixels, 32-pixel blocks
    int tiles_h, tiles_w, co_tiles;
    int HW, HWp, CG;           // window size, padded to even, channel groups of 8
    int XRS;                   // LDS entries per tile row (LW*Hf)
    int xbytes;                // bytes of the X region
    int tpr_shift;             // log2(threads per staged row)
    int L;                     // im2win row length Wi*Hf (materialised input)
};

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi)
{
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

template <bool FROM_WS>
__global__ __launch_bounds__(kThreads) void conv_f16_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ ws,
                                                            const uint16_t* __restrict__ w,
                                                            float* __restrict__ y, F16Args a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    uint4* X = reinterpret_cast<uint4*>(smem);
    uint4* Wl = reinterpret_cast<uint4*>(smem + a.xbytes);

    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co;
    const int sh = a.c.sh, sw = a.c.sw;
    const int Ho = a.c.Ho, Wo = a.c.Wo, Hf = a.c.Hf, Wf = a.c.Wf;
    const int HW = a.HW;

    int b = blockIdx.x;
    const int co_t = b % a.co_tiles; b /= a.co_tiles;
    const int tw_t = b % a.tiles_w;  b /= a.tiles_w;
    const int th_t = b % a.tiles_h;  b /= a.tiles_h;
    const int n = b;
    const int ho0 = th_t * a.TH, wo0 = tw_t * a.TW;
    const int co0 = co_t * kCoTile;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int wave = uniform(tid >> 6);

    int xoff[2];
    bool bok[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int pb = wave + 4 * m;
        bok[m] = pb < a.npb;
        int p = min(pb * 32 + l32, a.P - 1);
        const int th = p / a.TW, tw = p - (p / a.TW) * a.TW;
        xoff[m] = th * a.XRS + tw * sw * Hf + hl;
    }
    const int woff = hl * 64 + l32;

    floatx16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][m][r] = 0.f;

    const int tpr = 1 << a.tpr_shift;
    const int rsub = tid >> a.tpr_shift, csub = tid & (tpr - 1);
    const int rstep = kThreads >> a.tpr_shift;
    const int nsteps = a.HWp >> 1;
    const bool odd = (HW & 1) != 0;

    for (int g = 0; g < a.CG; ++g) {
        const int cb = 8 * g;
        __syncthreads();
        // ---- im2win rows of the tile, channels cb..cb+7 -> X -------------
        if (!FROM_WS) {
            const int64_t cstride = (int64_t)Hi * Wi;
            const int nrows = a.TH * Hf;
            const int ncol = min(a.LW, Wi - wo0 * sw);   // last column tile may be cut by Wi
            for (int r = rsub; r < nrows; r += rstep) {
                const int th = r / Hf, kh = r - (r / Hf) * Hf;
                if (ho0 + th >= Ho) continue;
                const uint16_t* gb =
                    x + (((int64_t)n * Ci + cb) * Hi + (ho0 + th) * sh + kh) * Wi + wo0 * sw;
                uint4* l = X + th * a.XRS + kh;
                for (int col = csub; col < ncol; col += tpr) {
                    uint16_t v[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) v[q] = cb + q < Ci ? gb[q * cstride + col] : 0;
                    l[col * Hf] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]),
                                             pack2(v[4], v[5]), pack2(v[6], v[7]));
                }
            }
        } else {
            const int64_t cstride = (int64_t)Ho * a.L;
            const int len = min(a.LW, Wi - wo0 * sw) * Hf;
            for (int r = rsub; r < a.TH; r += rstep) {
                if (ho0 + r >= Ho) continue;
                const uint16_t* gb =
                    ws + (((int64_t)n * Ci + cb) * Ho + ho0 + r) * a.L + wo0 * sw * Hf;
                uint4* l = X + r * a.XRS;
                for (int e = csub; e < len; e += tpr) {
                    uint16_t v[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) v[q] = cb + q < Ci ? gb[q * cstride + e] : 0;
                    l[e] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]),
                                      pack2(v[6], v[7]));
                }
            }
        }
        // ---- filters of channels cb..cb+7 in window order -> Wl ------------
        for (int idx = tid; idx < a.HWp * kCoTile; idx += kThreads) {
            const int j = idx >> 6, col = idx & 63;
            uint16_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (j < HW && co0 + col < Co) {
                const int kw = j / Hf, kh = j - (j / Hf) * Hf;
                const uint16_t* gw = w + ((int64_t)(co0 + col) * Ci + cb) * HW + kh * Wf + kw;
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = cb + q < Ci ? gw[q * HW] : 0;
            }
            Wl[idx] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]),
                                 pack2(v[6], v[7]));
        }
        __syncthreads();

        for (int t = 0; t < nsteps; ++t) {
            half8_t av[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 u = Wl[t * 128 + woff + i * 32];
                __builtin_memcpy(&av[i], &u, 16);
            }
            const bool zero_b = odd && hl && t == nsteps - 1;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                if (!bok[m]) continue;
                uint4 u = X[xoff[m] + 2 * t];
                if (zero_b) u = make_uint4(0, 0, 0, 0);
                half8_t bv;
                __builtin_memcpy(&bv, &u, 16);
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv, acc[i][m], 0, 0, 0);
            }
        }
    }

    // Output block (i, m): lane holds pixel l32 and channels 8*(r/4) + 4*hl + r%4.
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        if (!bok[m]) continue;
        const int p = (wave + 4 * m) * 32 + l32;
        if (p >= a.P) continue;
        const int th = p / a.TW, tw = p - (p / a.TW) * a.TW;
        const int ho = ho0 + th, wo = wo0 + tw;
        if (ho >= Ho || wo >= Wo) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = co0 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (co < Co) y[(((int64_t)n * Co + co) * Ho + ho) * Wo + wo] = acc[i][m][r];
            }
    }
}

// log2 of the smallest power of two >= v, but never above cap (cap >= 1):
// the result p satisfies 1 <= (1 << p) <= cap.
int log2_ceil_pow2(int v, int cap)
{
    int sh = 0;
    while ((1 << sh) < v && (2 << sh) <= cap) ++sh;
    return sh;
}

}  // namespace

int launch_conv_f16(const uint16_t* x, const uint16_t* ws, const uint16_t* w, float* y,
                    const ConvShape& c, hipStream_t stream)
{
    F16Args a;
    a.c = c;
    a.HW = c.Hf * c.Wf;
    a.HWp = (a.HW + 1) & ~1;
    a.CG = ceil_div(c.Ci, 8);
    const int wbytes = a.HWp * kCoTile * 16;
    a.TW = std::min(c.Wo, kPxTile);
    for (;;) {
        a.TH = std::max(1, std::min(c.Ho, kPxTile / a.TW));
        a.LW = (a.TW - 1) * c.sw + c.Wf;
        a.XRS = a.LW * c.Hf;
        while (a.TH > 1 && wbytes + a.TH * a.XRS * 16 > kMaxLds) --a.TH;
        if (wbytes + a.TH * a.XRS * 16 <= kMaxLds || a.TW == 1) break;
        a.TW = std::max(1, a.TW / 2);
    }
    a.xbytes = a.TH * a.XRS * 16;
    const size_t lds = (size_t)a.xbytes + wbytes;
    if (lds > kMaxLds) return -1;
    a.P = a.TH * a.TW;
    a.npb = ceil_div(a.P, 32);
    a.tiles_h = ceil_div(c.Ho, a.TH);
    a.tiles_w = ceil_div(c.Wo, a.TW);
    a.co_tiles = ceil_div(c.Co, kCoTile);
    a.L = c.Wi * c.Hf;
    a.tpr_shift = log2_ceil_pow2(ws ? a.LW * c.Hf : a.LW, kThreads);
    const int64_t blocks = (int64_t)c.N * a.tiles_h * a.tiles_w * a.co_tiles;
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    // Allow the full 160 KiB of gfx950 LDS.
    ensure_lds_limit(ws ? (const void*)conv_f16_kernel<true> : (const void*)conv_f16_kernel<false>,
                     kMaxLds);
    if (ws)
        hipLaunchKernelGGL(conv_f16_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), lds,
                           stream, x, ws, w, y, a);
    else
        hipLaunchKernelGGL(conv_f16_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), lds,
                           stream, x, ws, w, y, a);
    return launch_status();
}

}  // namespace im2win
