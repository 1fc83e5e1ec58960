// Fallback im2win convolution for shapes outside the tiled kernels' LDS
// envelope (very wide rows or very large filters). One thread per output;
// the window is read from the packed im2win tensor when one is given (one
// contiguous run of Wf*Hf per channel), else straight from x. Accumulates
// in fp32 with fused multiply-adds, channel by channel, in window order.
#include "common.hpp"
#include "kernels.hpp"

namespace im2win {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v)
{
    _Float16 h;
    __builtin_memcpy(&h, &v, 2);
    return (float)h;
}

template <typename T, bool FROM_WS>
__global__ __launch_bounds__(kThreads) void conv_generic_kernel(const T* __restrict__ x,
                                                                const T* __restrict__ ws,
                                                                const T* __restrict__ w,
                                                                float* __restrict__ y,
                                                                ConvShape c, int64_t total)
{
    const int64_t o = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (o >= total) return;
    const int wo = (int)(o % c.Wo);
    const int ho = (int)((o / c.Wo) % c.Ho);
    const int co = (int)((o / ((int64_t)c.Wo * c.Ho)) % c.Co);
    const int64_t n = o / ((int64_t)c.Wo * c.Ho * c.Co);
    const int HW = c.Hf * c.Wf;
    const int64_t L = (int64_t)c.Wi * c.Hf;
    float acc = 0.f;
    for (int ci = 0; ci < c.Ci; ++ci) {
        const T* wp = w + ((int64_t)co * c.Ci + ci) * HW;
        if (FROM_WS) {
            const T* win = ws + ((n * c.Ci + ci) * c.Ho + ho) * L + (int64_t)wo * c.sw * c.Hf;
            for (int kw = 0; kw < c.Wf; ++kw)
                for (int kh = 0; kh < c.Hf; ++kh)
                    acc = __builtin_fmaf(to_f32(win[kw * c.Hf + kh]), to_f32(wp[kh * c.Wf + kw]),
                                         acc);
        } else {
            const T* xp = x + ((n * c.Ci + ci) * c.Hi + (int64_t)ho * c.sh) * c.Wi + wo * c.sw;
            for (int kw = 0; kw < c.Wf; ++kw)
                for (int kh = 0; kh < c.Hf; ++kh)
                    acc = __builtin_fmaf(to_f32(xp[(int64_t)kh * c.Wi + kw]),
                                         to_f32(wp[kh * c.Wf + kw]), acc);
        }
    }
    y[o] = acc;
}

template <typename T>
int launch_generic(const T* x, const T* ws, const T* w, float* y, const ConvShape& c,
                   hipStream_t stream)
{
    const int64_t total = (int64_t)c.N * c.Co * c.Ho * c.Wo;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    if (ws)
        hipLaunchKernelGGL((conv_generic_kernel<T, true>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, stream, x, ws, w, y, c, total);
    else
        hipLaunchKernelGGL((conv_generic_kernel<T, false>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, stream, x, ws, w, y, c, total);
    return launch_status();
}

}  // namespace

int launch_conv_generic_f32(const float* x, const float* ws, const float* w, float* y,
                            const ConvShape& c, hipStream_t stream)
{
    return launch_generic<float>(x, ws, w, y, c, stream);
}

int launch_conv_generic_f16(const uint16_t* x, const uint16_t* ws, const uint16_t* w, float* y,
                            const ConvShape& c, hipStream_t stream)
{
    return launch_generic<uint16_t>(x, ws, w, y, c, stream);
}

}  // namespace im2win
