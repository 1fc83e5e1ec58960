// Rate probes: the dense arithmetic rates this chip sustains, measured, to
// read the convolution kernels' rates against (the published peaks assume
// the 2.4 GHz clock, which sustained matrix work does not hold).
//
// Each wave runs `iters` rounds of 4 independent operations of one kind on
// operands held in registers (no memory traffic inside the loop) and writes
// one float per lane so the work cannot be removed:
//  kind 0: v_fma_f32, 8 independent chains (the unpacked vector rate),
//  kind 1: v_mfma_f32_32x32x2_f32, 4 accumulators,
//  kind 2: v_mfma_f32_32x32x16_f16, 4 accumulators.
#include "common.hpp"
#include "im2win.h"
#include "kernels.hpp"

namespace im2win {

namespace {

constexpr int kProbeThreads = 256;

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void peak_probe_kernel(float* __restrict__ out,
                                                                   int iters)
{
    const int tid = threadIdx.x;
    const float seed = 1.0f + 1e-7f * (float)(tid & 63);
    float res = 0.f;
    if constexpr (KIND == 0) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = seed + (float)j;
        const float mul = 0.999999f, add = 1e-7f * seed;
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf(v[j], mul, add);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) res += v[j];
    } else if constexpr (KIND == 1) {
        floatx16_t acc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
        const float a = seed, b = 1.0f / seed;
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                acc[k] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) res += acc[k][r];
    } else {
        floatx16_t acc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
        half8_t a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = (_Float16)(seed * 0.5f);
            b[e] = (_Float16)(0.25f + 1e-3f * (float)e);
        }
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) res += acc[k][r];
    }
    out[(int64_t)blockIdx.x * kProbeThreads + tid] = res;
}

}  // namespace

}  // namespace im2win

extern "C" {

double im2win_peak_probe_flops(int kind, int blocks, int iters)
{
    if (kind < 0 || kind > 2 || blocks < 1 || iters < 1) return 0.0;
    const double waves = (double)blocks * (im2win::kProbeThreads / 64) * (double)iters;
    if (kind == 0) return waves * 64 * 4 * 8 * 2;        // lanes x rounds x chains x (mul + add)
    if (kind == 1) return waves * 4 * (32.0 * 32 * 2 * 2);   // 4 MFMAs of 32x32x2
    return waves * 4 * (32.0 * 32 * 16 * 2);                 // 4 MFMAs of 32x32x16
}

int im2win_peak_probe(int kind, int blocks, int iters, float* out, void* stream)
{
    if (kind < 0 || kind > 2 || blocks < 1 || iters < 1 || !out) return IM2WIN_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks), block(im2win::kProbeThreads);
    if (kind == 0)
        hipLaunchKernelGGL(im2win::peak_probe_kernel<0>, grid, block, 0, st, out, iters);
    else if (kind == 1)
        hipLaunchKernelGGL(im2win::peak_probe_kernel<1>, grid, block, 0, st, out, iters);
    else
        hipLaunchKernelGGL(im2win::peak_probe_kernel<2>, grid, block, 0, st, out, iters);
    const int rc = im2win::launch_status();
    return rc == 0 ? IM2WIN_OK : IM2WIN_ELAUNCH;
}

}  // extern "C"
