// im2win for NHWC tensors (x: N x Hi x Wi x Ci, y: N x Ho x Wo x Co).
//
// The transform of "Im2win: Memory Efficient Convolution On SIMD
// Architectures" (Abstract: a row of windows flattened into one row) with
// the channels innermost:
//     ws[n][ho][w][kh][c] = x[n][ho*sh + kh][w][c],
// so the window of output (ho, wo) is the one contiguous run of Wf*Hf*Ci
// elements at wo*sw*Hf*Ci in row (n, ho), ordered (kw, kh, c). The
// convolution packs each column's Hf*Ci run into `pitch` elements, Hf*Ci
// rounded up to 32 bytes with zeros after it (no padding when Ci*elem is a
// multiple of 32): every 32-byte K slice of a window is then contiguous and
// aligned, whatever Ci and the strides, at the cost of multiplying the zeros.
//
//  * pack_nhwc_kernel: the transform, unpadded (16-byte chunks when Ci*elem
//    is a multiple of 16, elements otherwise).
//  * pack_nhwc_pad_kernel: the transform with runs padded to the pitch.
//  * filter_khwc_kernel: filters reordered to the window order, padded the
//    same way: wr[co][kw*pitch + kh*Ci + c] = w[co][c][kh][kw], zero past
//    Hf*Ci in each run.
//  * conv_direct_nhwc_kernel: one thread per output, channels of an output
//    pixel in consecutive lanes (they share its window).
// The convolution over the packed tensor is the matrix-core GEMM of
// im2col.hip, fed with these overlapping window rows.
#include "common.hpp"
#include "kernels.hpp"

namespace im2win {

namespace {

template <typename V>
__global__ __launch_bounds__(256) void pack_nhwc_kernel(const V* __restrict__ x, V* __restrict__ ws,
                                                        ConvShape c, int cv, int64_t total)
{
    // cv = Ci in units of V; element e = ((((n*Ho + ho)*Wi + w)*Hf + kh)*cv + cc.
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    int64_t r = e / cv;
    const int cc = (int)(e - r * cv);
    const int kh = (int)(r % c.Hf);
    r /= c.Hf;
    const int w = (int)(r % c.Wi);
    r /= c.Wi;
    const int ho = (int)(r % c.Ho);
    const int64_t n = r / c.Ho;
    ws[e] = x[((n * c.Hi + (int64_t)ho * c.sh + kh) * c.Wi + w) * cv + cc];
}

// The transform with each column's run padded: chunk e (16 bytes, P
// elements) of ws = elements e*P .. e*P+P-1 of the rows of `pitch`
// elements, ws[((n*Ho + ho)*Wi + w)*pitch + kh*Ci + c] = x[n][ho*sh + kh][w][c]
// and zero from Hf*Ci on. pitch is a multiple of P.
template <typename T>
__global__ __launch_bounds__(256) void pack_nhwc_pad_kernel(const T* __restrict__ x,
                                                            uint4* __restrict__ ws, ConvShape c,
                                                            int pitch, int64_t total)
{
    constexpr int P = 16 / (int)sizeof(T);
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    const int64_t run = e * P / pitch;
    const int j0 = (int)(e * P - run * pitch);
    const int w = (int)(run % c.Wi);
    const int64_t r = run / c.Wi;
    const int ho = (int)(r % c.Ho);
    const int64_t n = r / c.Ho;
    const int HC = c.Hf * c.Ci;
    T v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int j = j0 + i;
        T t = 0;
        if (j < HC) {
            const int kh = j / c.Ci, cc = j - kh * c.Ci;
            t = x[((n * c.Hi + (int64_t)ho * c.sh + kh) * c.Wi + w) * c.Ci + cc];
        }
        v[i] = t;
    }
    uint4 o;
    __builtin_memcpy(&o, v, 16);
    ws[e] = o;
}

template <typename T>
__global__ __launch_bounds__(256) void filter_khwc_kernel(const T* __restrict__ w,
                                                          T* __restrict__ wr, ConvShape c,
                                                          int pitch)
{
    const int64_t K = (int64_t)c.Wf * pitch;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)c.Co * K) return;
    const int co = (int)(e / K);
    const int k = (int)(e - (int64_t)co * K);
    const int kw = k / pitch, j = k - kw * pitch;
    T t = 0;
    if (j < c.Hf * c.Ci) {
        const int kh = j / c.Ci, ci = j - kh * c.Ci;
        t = w[(((int64_t)co * c.Ci + ci) * c.Hf + kh) * c.Wf + kw];
    }
    wr[e] = t;
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v)
{
    _Float16 h;
    __builtin_memcpy(&h, &v, 2);
    return (float)h;
}

template <typename T>
__global__ __launch_bounds__(256) void conv_direct_nhwc_kernel(const T* __restrict__ x,
                                                               const T* __restrict__ w,
                                                               float* __restrict__ y, ConvShape c,
                                                               int64_t total)
{
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= total) return;
    const int co = (int)(o % c.Co);
    const int64_t q = o / c.Co;
    const int wo = (int)(q % c.Wo);
    const int ho = (int)((q / c.Wo) % c.Ho);
    const int64_t n = q / ((int64_t)c.Wo * c.Ho);
    const T* wp = w + (int64_t)co * c.Ci * c.Hf * c.Wf;
    float acc = 0.f;
    // Same term order as the NCHW kernels: channel, then kh, then kw.
    for (int ci = 0; ci < c.Ci; ++ci)
        for (int kh = 0; kh < c.Hf; ++kh) {
            const T* xr = x + ((n * c.Hi + (int64_t)ho * c.sh + kh) * c.Wi + (int64_t)wo * c.sw) * c.Ci + ci;
            for (int kw = 0; kw < c.Wf; ++kw)
                acc = __builtin_fmaf(to_f32(xr[(int64_t)kw * c.Ci]),
                                     to_f32(wp[((int64_t)ci * c.Hf + kh) * c.Wf + kw]), acc);
        }
    y[o] = acc;
}

}  // namespace

int launch_pack_nhwc(const void* x, void* ws, const ConvShape& c, int elem, hipStream_t stream)
{
    const int64_t elems = (int64_t)c.N * c.Ho * c.Wi * c.Hf * c.Ci;
    const bool vec = ((int64_t)c.Ci * elem) % 16 == 0 && (uintptr_t)x % 16 == 0 &&
                     (uintptr_t)ws % 16 == 0;
    const int per = vec ? 16 / elem : 1;
    const int64_t total = elems / per;
    const int64_t blocks = (total + 255) / 256;
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    const int cv = c.Ci / per;
    if (vec)
        hipLaunchKernelGGL(pack_nhwc_kernel<uint4>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint4*)x, (uint4*)ws, c, cv, total);
    else if (elem == 2)
        hipLaunchKernelGGL(pack_nhwc_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint16_t*)x, (uint16_t*)ws, c, cv, total);
    else
        hipLaunchKernelGGL(pack_nhwc_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint32_t*)x, (uint32_t*)ws, c, cv, total);
    return launch_status();
}

int nhwc_pitch(const ConvShape& c, int elem)
{
    const int q = 32 / elem;
    return (c.Hf * c.Ci + q - 1) / q * q;
}

int launch_pack_nhwc_padded(const void* x, void* ws, const ConvShape& c, int elem,
                            hipStream_t stream)
{
    const int pitch = nhwc_pitch(c, elem);
    if (pitch == c.Hf * c.Ci) return launch_pack_nhwc(x, ws, c, elem, stream);
    if ((uintptr_t)ws % 16 != 0) return -1;
    const int64_t total = (int64_t)c.N * c.Ho * c.Wi * pitch * elem / 16;
    const int64_t blocks = (total + 255) / 256;
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    if (elem == 2)
        hipLaunchKernelGGL(pack_nhwc_pad_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, (const uint16_t*)x, (uint4*)ws, c, pitch, total);
    else
        hipLaunchKernelGGL(pack_nhwc_pad_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, (const uint32_t*)x, (uint4*)ws, c, pitch, total);
    return launch_status();
}

int launch_filter_khwc(const void* w, void* wr, const ConvShape& c, int elem, hipStream_t stream)
{
    const int pitch = nhwc_pitch(c, elem);
    const int64_t total = (int64_t)c.Co * c.Wf * pitch;
    const int64_t blocks = (total + 255) / 256;
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    if (elem == 2)
        hipLaunchKernelGGL(filter_khwc_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint16_t*)w, (uint16_t*)wr, c, pitch);
    else
        hipLaunchKernelGGL(filter_khwc_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint32_t*)w, (uint32_t*)wr, c, pitch);
    return launch_status();
}

int launch_conv_direct_nhwc(const void* x, const void* w, float* y, const ConvShape& c, int elem,
                            hipStream_t stream)
{
    const int64_t total = (int64_t)c.N * c.Ho * c.Wo * c.Co;
    const int64_t blocks = (total + 255) / 256;
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    if (elem == 2)
        hipLaunchKernelGGL(conv_direct_nhwc_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, (const uint16_t*)x, (const uint16_t*)w, y, c, total);
    else
        hipLaunchKernelGGL(conv_direct_nhwc_kernel<float>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, (const float*)x, (const float*)w, y, c, total);
    return launch_status();
}

}  // namespace im2win
