// im2col + GEMM convolution: the memory-hungry baseline that "Enabling
// Memory-efficient Im2win Convolution with Multi-precision Support on GPU
// CUDA and Tensor Cores" compares im2win against (Fig. 1, right: every
// window unfolded into its own column; Abstract: GEMM-based convolution).
//
//  * im2col_kernel writes, for every output pixel q = (n*Ho + ho)*Wo + wo, its
//    receptive field as one row of K = Ci*Hf*Wf elements in (ci, kh, kw)
//    order, zero-padded to KP elements (a multiple of 32 bytes: one GEMM
//    slice, 16 halves or 8 floats):
//        col[q][(ci*Hf + kh)*Wf + kw] = x[n][ci][ho*sh + kh][wo*sw + kw].
//    That is the transpose of the usual K x P layout, with the same size; it
//    makes each MFMA operand slice one contiguous 16-byte load.
//  * filter_pad_kernel copies the filters into rows of KP (zero tail).
//  * gemm_nt_kernel computes y[n][co][p] = sum_k w[co][k] * col[q][k] on the
//    matrix cores with the same instructions as the im2win kernels
//    (v_mfma_f32_32x32x16_f16, v_mfma_f32_32x32x2_f32): a wave owns 64
//    output channels x 64 pixels (2 x 2 tiles of 32 x 32), operands come
//    straight from memory (16 bytes per lane per slice), the next slice is
//    loaded while the current one is multiplied.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace im2win {

namespace {

constexpr int kGemmThreads = 256;   // 4 waves: 64 channels x 256 pixels per workgroup

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gbuf(const void* base, uint64_t bytes)
{
    const uint32_t n = bytes >= 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

struct ColArgs {
    ConvShape c;
    int K, KP;
    int64_t rows;   // N*Ho*Wo
};

template <typename T>
__global__ __launch_bounds__(256) void im2col_kernel(const T* __restrict__ x, T* __restrict__ col,
                                                    ColArgs a)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= a.rows * a.KP) return;
    const int64_t q = e / a.KP;
    const int k = (int)(e - q * a.KP);
    T v = 0;
    if (k < a.K) {
        const int HW = a.c.Hf * a.c.Wf;
        const int ci = k / HW, r = k - ci * HW;
        const int kh = r / a.c.Wf, kw = r - kh * a.c.Wf;
        const int64_t plane = (int64_t)a.c.Ho * a.c.Wo;
        const int64_t n = q / plane;
        const int pix = (int)(q - n * plane);
        const int ho = pix / a.c.Wo, wo = pix - ho * a.c.Wo;
        v = x[(((n * a.c.Ci + ci) * a.c.Hi) + (int64_t)ho * a.c.sh + kh) * a.c.Wi +
              (int64_t)wo * a.c.sw + kw];
    }
    col[e] = v;
}

template <typename T>
__global__ __launch_bounds__(256) void filter_pad_kernel(const T* __restrict__ w, T* __restrict__ wp,
                                                         int Co, int K, int KP)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)Co * KP) return;
    const int co = (int)(e / KP), k = (int)(e - (int64_t)co * KP);
    wp[e] = k < K ? w[(int64_t)co * K + k] : T(0);
}

struct GemmArgs {
    int Co, KP, P;            // channels, K per row (a multiple of the slice), pixels per image
    int64_t rows;             // N*P
    uint64_t colbytes, wbytes, ybytes;
    // Rows of the B matrix: im2col rows (q*KP), or the overlapping window runs
    // of an NHWC im2win tensor (((n*Ho + ho)*Wi + wo*sw)*HfC). Output NCHW or NHWC.
    bool win_rows, y_nhwc;
    int Ho, Wo, Wi, sw, HfC;
};

// One MFMA slice: fp16 16 K values (lanes 0-31 the first 8, 32-63 the next 8),
// fp32 8 K values over four 32x32x2 steps (lane half hl holds k0 + 4*hl + j
// for step j). A and B use the same mapping, so the sum covers each k once.
template <bool F16>
__global__ __launch_bounds__(kGemmThreads) void gemm_nt_kernel(const void* __restrict__ colv,
                                                               const void* __restrict__ wv,
                                                               float* __restrict__ y, GemmArgs a)
{
    constexpr int E = F16 ? 2 : 4;             // element bytes
    constexpr int SK = F16 ? 16 : 8;           // K values per slice
    const int lane = threadIdx.x & 63, hl = lane >> 5, l32 = lane & 31;
    const int wave = uniform(threadIdx.x >> 6);
    const int co_tiles = (a.Co + 63) / 64;
    const int co0 = (int)(blockIdx.x % co_tiles) * 64;
    const int64_t q0 = (int64_t)(blockIdx.x / co_tiles) * 256 + wave * 64;

    const __amdgpu_buffer_rsrc_t rc = gbuf(colv, a.colbytes);
    const __amdgpu_buffer_rsrc_t rw = gbuf(wv, a.wbytes);
    const uint32_t kMissOff = 0xFFFFFFF0u;
    // Byte offsets of this lane's operand rows (missing rows read zeros).
    uint32_t ao[2], bo[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int co = co0 + i * 32 + l32;
        ao[i] = co < a.Co ? (uint32_t)(((int64_t)co * a.KP + (SK / 2) * hl) * E) : kMissOff;
        const int64_t q = q0 + i * 32 + l32;
        int64_t row = q * a.KP;
        if (a.win_rows) {
            const int64_t n = q / a.P;
            const int pix = (int)(q - n * a.P);
            const int ho = pix / a.Wo, wo = pix - ho * a.Wo;
            row = ((n * a.Ho + ho) * a.Wi + (int64_t)wo * a.sw) * a.HfC;
        }
        const uint64_t b = (uint64_t)(row + (SK / 2) * hl) * E;
        bo[i] = q < a.rows && b < 0xFFFFFFF0ull ? (uint32_t)b : kMissOff;
    }

    floatx16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    uint4 A[2], B[2], An[2], Bn[2];
    auto load = [&](uint4* Ad, uint4* Bd, int k0) {
        const uint32_t ko = (uint32_t)k0 * E;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const auto va = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(ao[i] == kMissOff ? kMissOff : ao[i] + ko), 0, 0);
            const auto vb = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(bo[i] == kMissOff ? kMissOff : bo[i] + ko), 0, 0);
            Ad[i] = make_uint4(va[0], va[1], va[2], va[3]);
            Bd[i] = make_uint4(vb[0], vb[1], vb[2], vb[3]);
        }
    };
    auto mma = [&](const uint4* Ad, const uint4* Bd) {
        if constexpr (F16) {
            half8_t ah[2], bh[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                __builtin_memcpy(&ah[i], &Ad[i], 16);
                __builtin_memcpy(&bh[i], &Bd[i], 16);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bh[j], acc[i][j], 0, 0, 0);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                float af[2], bf[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint32_t ua = s == 0 ? Ad[i].x : s == 1 ? Ad[i].y : s == 2 ? Ad[i].z : Ad[i].w;
                    const uint32_t ub = s == 0 ? Bd[i].x : s == 1 ? Bd[i].y : s == 2 ? Bd[i].z : Bd[i].w;
                    af[i] = __uint_as_float(ua);
                    bf[i] = __uint_as_float(ub);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bf[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    const int nsl = a.KP / SK;   // KP is a multiple of SK
    load(A, B, 0);
    for (int t = 0; t < nsl; ++t) {
        if (t + 1 < nsl) load(An, Bn, (t + 1) * SK);
        mma(A, B);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            A[i] = An[i];
            B[i] = Bn[i];
        }
    }

    // Output: lane holds pixel l32 of each block and channels
    // 8*(r/4) + 4*hl + r%4 of each 32-channel block.
    const __amdgpu_buffer_rsrc_t ry = gbuf(y, a.ybytes);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t q = q0 + j * 32 + l32;
        if (q >= a.rows) continue;
        const int64_t n = q / a.P;
        const int p = (int)(q - n * a.P);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = co0 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
                const int64_t off = a.y_nhwc ? q * a.Co + co : (n * a.Co + co) * a.P + p;
                if (co < a.Co)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), ry,
                                                          (int)(off * 4), 0, 0);
            }
    }
}

int launch_gemm(const void* b, const void* a, float* y, const GemmArgs& g, int Co, int elem,
                hipStream_t stream)
{
    // 32-bit buffer offsets: the chunk's matrix and output below 4 GiB.
    if (g.colbytes >= 0xFFFFFFF0ull || g.ybytes >= 0xFFFFFFF0ull || g.wbytes >= 0xFFFFFFF0ull)
        return -1;
    const int64_t blocks = ((g.rows + 255) / 256) * ((Co + 63) / 64);
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    if (elem == 2)
        hipLaunchKernelGGL(gemm_nt_kernel<true>, dim3((unsigned)blocks), dim3(kGemmThreads), 0,
                           stream, b, a, y, g);
    else
        hipLaunchKernelGGL(gemm_nt_kernel<false>, dim3((unsigned)blocks), dim3(kGemmThreads), 0,
                           stream, b, a, y, g);
    return launch_status();
}

int64_t padded_k(const ConvShape& c, int elem)
{
    const int64_t K = (int64_t)c.Ci * c.Hf * c.Wf;
    const int64_t step = 32 / elem;   // one slice of the GEMM
    return (K + step - 1) / step * step;
}

}  // namespace

size_t im2col_row_elems(const ConvShape& c, int elem) { return (size_t)padded_k(c, elem); }

int launch_im2col(const void* x, void* col, const ConvShape& c, int elem, hipStream_t stream)
{
    ColArgs a;
    a.c = c;
    a.K = c.Ci * c.Hf * c.Wf;
    a.KP = (int)padded_k(c, elem);
    a.rows = (int64_t)c.N * c.Ho * c.Wo;
    const int64_t total = a.rows * a.KP;
    const int64_t blocks = (total + 255) / 256;
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    if (elem == 2)
        hipLaunchKernelGGL(im2col_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint16_t*)x, (uint16_t*)col, a);
    else
        hipLaunchKernelGGL(im2col_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint32_t*)x, (uint32_t*)col, a);
    return launch_status();
}

int launch_im2col_gemm(const void* col, const void* w, void* wpad, float* y, const ConvShape& c,
                       int elem, hipStream_t stream)
{
    const int K = c.Ci * c.Hf * c.Wf;
    const int KP = (int)padded_k(c, elem);
    const int64_t wtotal = (int64_t)c.Co * KP;
    const int64_t wblocks = (wtotal + 255) / 256;
    if (wblocks > 0x7fffffff) return -1;
    if (elem == 2)
        hipLaunchKernelGGL(filter_pad_kernel<uint16_t>, dim3((unsigned)wblocks), dim3(256), 0, stream,
                           (const uint16_t*)w, (uint16_t*)wpad, c.Co, K, KP);
    else
        hipLaunchKernelGGL(filter_pad_kernel<uint32_t>, dim3((unsigned)wblocks), dim3(256), 0, stream,
                           (const uint32_t*)w, (uint32_t*)wpad, c.Co, K, KP);
    GemmArgs g{};
    g.Co = c.Co;
    g.KP = KP;
    g.P = c.Ho * c.Wo;
    g.rows = (int64_t)c.N * g.P;
    g.colbytes = (uint64_t)g.rows * KP * elem;
    g.wbytes = (uint64_t)wtotal * elem;
    g.ybytes = (uint64_t)g.rows * c.Co * 4;
    g.win_rows = false;
    g.y_nhwc = false;
    return launch_gemm(col, wpad, y, g, c.Co, elem, stream);
}

bool nhwc_gemm_applies(const ConvShape& c, int elem)
{
    // Window runs of whole slices (K = Wf*Hf*Ci), each slice 16 aligned bytes.
    return c.Ci % (elem == 2 ? 16 : 8) == 0;
}

int launch_nhwc_gemm(const void* ws, const void* wr, float* y, const ConvShape& c, int elem,
                     hipStream_t stream)
{
    if (!nhwc_gemm_applies(c, elem)) return -1;
    GemmArgs g{};
    g.Co = c.Co;
    g.HfC = c.Hf * c.Ci;
    g.KP = c.Wf * g.HfC;
    g.P = c.Ho * c.Wo;
    g.rows = (int64_t)c.N * g.P;
    g.colbytes = (uint64_t)c.N * c.Ho * c.Wi * g.HfC * elem;
    g.wbytes = (uint64_t)c.Co * g.KP * elem;
    g.ybytes = (uint64_t)g.rows * c.Co * 4;
    g.win_rows = true;
    g.y_nhwc = true;
    g.Ho = c.Ho;
    g.Wo = c.Wo;
    g.Wi = c.Wi;
    g.sw = c.sw;
    return launch_gemm(ws, wr, y, g, c.Co, elem, stream);
}

}  // namespace im2win
