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

}  // namespace im2win
