// Shared helpers for the im2win HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace im2win {

// Unsigned division by a runtime-invariant divisor d >= 1 for dividends
// n < 2^31, by multiply-high and shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, floor(n / d) = (mulhi(n, m) + n) >> l.
struct FastDiv {
    uint32_t d, m, l;
    FastDiv() : d(1), m(1), l(0) {}
    explicit FastDiv(uint32_t dv) : d(dv) {
        l = 0;
        while ((1ull << l) < dv) ++l;
        m = (uint32_t)(((1ull << 32) * ((1ull << l) - dv)) / dv + 1);
    }
    __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
        uint32_t hi = (uint32_t)(((uint64_t)n * m) >> 32);
        return (uint32_t)(((uint64_t)hi + n) >> l);
    }
};

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// Wave-uniform value in an SGPR (the argument must already be uniform).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Tile of workgroup b of a grid of `grid`. Workgroups are handed to the 8
// XCDs in turn (b on XCD b % 8). grouped: XCD x takes the contiguous tiles
// [x*G8, (x+1)*G8) of the first 8*G8 (G8 = grid / 8), so neighbouring tiles,
// which share input rows, share that XCD's L2; the last partial round keeps
// launch order. Otherwise tile = b (launch order).
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t grid, bool grouped)
{
    if (!grouped) return b;
    const int64_t G8 = grid / 8;
    return b < 8 * G8 ? (b % 8) * G8 + b / 8 : b;
}

// Raw buffer resource over [base, base + bytes): a load at a byte offset
// (vector + scalar) at or past `bytes` returns zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes per lane from buffer r at vector offset voff straight into LDS at
// byte lds + 16*lane (buffer_load_dwordx4 ... lds; lds wave-uniform, M0
// saved and restored around the load). An out-of-range lane writes zeros.
// The load counts in vmcnt like any other vector load.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff)
{
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(voff), "s"(r)
        : "memory");
}

// Waits until at most N of this wave's vector loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace im2win
