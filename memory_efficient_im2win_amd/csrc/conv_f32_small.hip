// fp32 im2win convolution for problems too small to fill the chip with
// output tiles (one image of a late layer, a few hundred output pixels), on
// the CDNA4 matrix cores (v_mfma_f32_16x16x4_f32).
//
// The single-precision path of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract: full
// precision; Fig. 1: each output is the dot product of a filter with its
// im2win window) for shapes whose 32 x 32 output tiles number fewer than the
// chip's 256 compute units. Such a call is bound by latency, not by
// arithmetic or bytes, so the kernel is built to wait for memory once:
//
//  * GEMM view: rows = output channels (A = filters), columns = output
//    pixels of one image (B = windows), K = (input channel, kh, kw) in the
//    filter's memory order. A workgroup owns 16 channels x 32 consecutive
//    pixels of one image (two 16 x 16 blocks), so the grid has four times
//    as many workgroups as 32 x 32 tiles would give.
//  * One stage: the workgroup copies the input rows its pixels' windows
//    cover (every input channel) into LDS, with a table of each K index's
//    LDS offset; at the same time each lane loads all the filter values it
//    will use straight from global memory into registers. Nothing is loaded
//    after the MFMAs start.
//  * The 8 waves split K: wave v takes a contiguous range of 16-index chunks.
//    In chunk q, sub-step s, the MFMA's four K slots are the indices
//    16q + 4g + s (g = lane group 0..3), so lane (i, g) holds the four
//    consecutive filter taps 16q + 4g .. +3 of channel co0 + i in one
//    16-byte register and reads the matching window value from LDS.
//  * Indices past K have a zero filter value and read a zero LDS entry, so
//    an infinity in a window never meets a padded tap.
//  * The 8 waves' partial sums go through LDS and are added in wave order
//    (0 + 1 + ... + 7) by the thread that stores the output: no atomics, the
//    same bits on every run.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "knobs.hpp"

namespace im2win {

namespace {

constexpr int kNW = 8;                    // waves per workgroup (K shares)
constexpr int kNT = 64 * kNW;
constexpr int kCoT = 16;                  // output channels per tile
constexpr int kPx = 32;                   // pixels per tile (two 16-pixel blocks)
constexpr int kLds = 160 * 1024;
constexpr uint32_t kMiss = 0xFFFFFFF0u;   // offset past every accepted buffer
constexpr int kCpw[] = {4, 8, 12, 16, 20, 24};   // built chunks-per-wave bounds

struct SArgs {
    ConvShape c;
    int K, KC;                // taps per filter, 16-index chunks (ceil(K / 16))
    int co_tiles, pt_img;     // channel tiles; pixel tiles per image
    int RIN;                  // input rows per channel in LDS
    int xent;                 // LDS entries of the rows (Ci*RIN*Wi); entry xent is zero
    int xq;                   // 16-byte chunks of the rows (vector copy)
    uint32_t toff;            // LDS byte offset of the K table
    uint32_t lds_bytes;
    uint32_t xbytes, wbytes, ybytes;
    bool swz;                 // XCD-grouped tile order
    FastDiv divWo, divWi, divWq, divRIN, divHW, divWf;
};


// CPW: chunks per wave at most; AVEC: K % 4 == 0 (16-byte filter loads);
// XVEC: Wi % 4 == 0 (16-byte row copies).
template <int CPW, bool AVEC, bool XVEC>
__global__ __launch_bounds__(kNT) void conv_f32_small_kernel(const float* __restrict__ x,
                                                             const float* __restrict__ w,
                                                             float* __restrict__ y, SArgs a)
{
    extern __shared__ __align__(16) float lds[];
    float* X = lds;
    const int* T = reinterpret_cast<const int*>(reinterpret_cast<const unsigned char*>(lds) + a.toff);

    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co;
    const int Hf = a.c.Hf, Wf = a.c.Wf, sh = a.c.sh, sw = a.c.sw;
    const int Ho = a.c.Ho, Wo = a.c.Wo;
    const int K = a.K, RIN = a.RIN;
    const int plane = Ho * Wo;

    // Tiles numbered pixel tile fastest, so the workgroups one XCD takes
    // (XCD-grouped order) share a few channel tiles: each XCD's L2 then holds
    // a slice of the filter instead of all of it.
    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x, a.swz);
    const int pts = a.c.N * a.pt_img;
    const int co_t = (int)(bid / pts);
    const int rest = (int)(bid - (int64_t)co_t * pts);
    const int n = rest / a.pt_img;
    const int pt = rest - n * a.pt_img;
    const int co0 = co_t * kCoT;
    const int p0 = pt * kPx;
    const int pend = min(p0 + kPx, plane);
    const int ho0 = (int)a.divWo.div((uint32_t)p0);
    const int hol = (int)a.divWo.div((uint32_t)(pend - 1));
    const int row0 = ho0 * sh;
    const int nrows = min((hol - ho0) * sh + Hf, Hi - row0);   // real rows, <= RIN

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int g = lane >> 4, j = lane & 15;

    // ---- filter values of this wave's chunks [qa, qb), into registers ------
    const int qa = wave * a.KC / kNW, qb = (wave + 1) * a.KC / kNW;
    const __amdgpu_buffer_rsrc_t wr = raw_rsrc(w, a.wbytes);
    const bool co_ok = co0 + j < Co;
    const uint32_t rowoff = (uint32_t)(co0 + j) * (uint32_t)K * 4;
    float av[CPW][4];
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
        const int k0 = 16 * (qa + q) + 4 * g;
        const bool live = qa + q < qb && co_ok;
        if (AVEC) {
            // K % 4 == 0: the four taps are all real or all past K.
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(
                wr, (int)(live && k0 < K ? rowoff + (uint32_t)k0 * 4 : kMiss), 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) av[q][e] = __uint_as_float(v[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                av[q][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    wr, (int)(live && k0 + e < K ? rowoff + (uint32_t)(k0 + e) * 4 : kMiss), 0, 0));
        }
    }

    // ---- input rows row0 .. row0 + nrows - 1 of every channel -> LDS --------
    // Entry (c*RIN + r)*Wi + col; rows past nrows are not written (no pixel of
    // the tile reads them).
    const __amdgpu_buffer_rsrc_t xr = raw_rsrc(x, a.xbytes);
    const int64_t img = (int64_t)n * Ci * Hi * Wi;
    if (XVEC) {
        const int wq = Wi >> 2;
        for (int e0 = 0; e0 < a.xq; e0 += 8 * kNT) {
            uint4 v[8];
            int dst[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = e0 + u * kNT + tid;
                const int row = (int)a.divWq.div((uint32_t)e);
                const int cq = e - row * wq;
                const int c = (int)a.divRIN.div((uint32_t)row);
                const int r = row - c * RIN;
                const bool ok = e < a.xq && r < nrows;
                dst[u] = ok ? row * Wi + 4 * cq : -1;
                const uint32_t off =
                    ok ? (uint32_t)((img + ((int64_t)c * Hi + row0 + r) * Wi + 4 * cq) * 4) : kMiss;
                const auto t = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)off, 0, 0);
                v[u] = make_uint4(t[0], t[1], t[2], t[3]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (dst[u] >= 0) *reinterpret_cast<uint4*>(X + dst[u]) = v[u];
        }
    } else {
        for (int e0 = 0; e0 < a.xent; e0 += 8 * kNT) {
            uint32_t v[8];
            int dst[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = e0 + u * kNT + tid;
                const int row = (int)a.divWi.div((uint32_t)e);
                const int col = e - row * Wi;
                const int c = (int)a.divRIN.div((uint32_t)row);
                const int r = row - c * RIN;
                const bool ok = e < a.xent && r < nrows;
                dst[u] = ok ? e : -1;
                const uint32_t off =
                    ok ? (uint32_t)((img + ((int64_t)c * Hi + row0 + r) * Wi + col) * 4) : kMiss;
                v[u] = __builtin_amdgcn_raw_buffer_load_b32(xr, (int)off, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (dst[u] >= 0) X[dst[u]] = __uint_as_float(v[u]);
        }
    }
    // K table: LDS entry of tap k = (c, kh, kw) from a pixel's window corner;
    // indices past K point at the zero entry.
    {
        int* Tw = const_cast<int*>(T);
        const int HW = Hf * Wf;
        for (int k = tid; k < 16 * a.KC; k += kNT) {
            int t = a.xent;
            if (k < K) {
                const int c = (int)a.divHW.div((uint32_t)k), rem = k - c * HW;
                const int kh = (int)a.divWf.div((uint32_t)rem), kw = rem - kh * Wf;
                t = (c * RIN + kh) * Wi + kw;
            }
            Tw[k] = t;
        }
        if (tid == 0) X[a.xent] = 0.f;
    }
    __syncthreads();

    // ---- MFMAs ------------------------------------------------------------
    int pix[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int p = min(p0 + 16 * b + j, pend - 1);
        const int ho = (int)a.divWo.div((uint32_t)p);
        const int wo = p - ho * Wo;
        pix[b] = (ho - ho0) * sh * Wi + wo * sw;
    }
    floatx4_t acc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    const int4* T4 = reinterpret_cast<const int4*>(T);
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
        if (qa + q < qb) {
            const int4 t = T4[(qa + q) * 4 + g];
            const int ts[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q][s], X[pix[b] + ts[s]],
                                                                 acc[b], 0, 0, 0);
            }
        }
    }

    // ---- fixed-order sum of the waves' shares, store -------------------------
    // Lane l of block b holds channel co0 + 4*(l/16) + r, pixel p0 + 16b + l%16
    // in acc[b][r].
    __syncthreads();   // every wave is done reading the rows
    float* red = lds;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * 2 + b) * 4 + r) * 64 + lane] = acc[b][r];
    __syncthreads();
    {
        const int b = tid >> 8, r = (tid >> 6) & 3, l = tid & 63;
        float s = red[((0 * 2 + b) * 4 + r) * 64 + l];
#pragma unroll
        for (int v = 1; v < kNW; ++v) s += red[((v * 2 + b) * 4 + r) * 64 + l];
        const int co = co0 + 4 * (l >> 4) + r;
        const int p = p0 + 16 * b + (l & 15);
        if (co < Co && p < pend) {
            const __amdgpu_buffer_rsrc_t yr = raw_rsrc(y, a.ybytes);
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(s), yr, (int)((((int64_t)n * Co + co) * plane + p) * 4), 0, 0);
        }
    }
}

// Plans a launch; false if the shape is outside the kernel's envelope:
// K at most 8 waves x 24 chunks of 16, the rows of a tile and the K table in
// LDS, tensors addressable with 32-bit buffer offsets.
bool plan(const ConvShape& c, SArgs& a, int& cpw)
{
    a.c = c;
    a.K = c.Ci * c.Hf * c.Wf;
    a.KC = ceil_div(a.K, 16);
    cpw = 0;
    for (int v : kCpw)
        if (v >= ceil_div(a.KC, kNW)) {   // the largest share is ceil(KC / 8)
            cpw = v;
            break;
        }
    if (!cpw) return false;
    const int plane = c.Ho * c.Wo;
    a.pt_img = ceil_div(plane, kPx);
    a.co_tiles = ceil_div(c.Co, kCoT);
    // Output rows a tile touches: at most (kPx - 1) / Wo + 2, never more than Ho.
    const int span = std::min(c.Ho, (kPx - 1) / c.Wo + 2);
    a.RIN = (span - 1) * c.sh + c.Hf;
    const int64_t xent = (int64_t)c.Ci * a.RIN * c.Wi;
    const int64_t xbytes_l = std::max<int64_t>((xent + 1) * 4, (int64_t)kNW * 2 * 4 * 64 * 4);
    const int64_t toff = (xbytes_l + 15) / 16 * 16;
    const int64_t lds = toff + (int64_t)16 * a.KC * 4;
    if (lds > kLds) return false;
    const int64_t xb = (int64_t)c.N * c.Ci * c.Hi * c.Wi * 4;
    const int64_t wb = (int64_t)c.Co * a.K * 4;
    const int64_t yb = (int64_t)c.N * c.Co * plane * 4;
    if (xb >= (int64_t)kMiss || wb >= 0x7fffffff || yb >= 0x7fffffff) return false;
    if ((int64_t)a.co_tiles * c.N * a.pt_img > 0x7fffffff) return false;
    a.xent = (int)xent;
    a.xq = (int)(xent / 4);
    a.toff = (uint32_t)toff;
    a.lds_bytes = (uint32_t)lds;
    a.xbytes = (uint32_t)xb;
    a.wbytes = (uint32_t)wb;
    a.ybytes = (uint32_t)yb;
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divWi = FastDiv((uint32_t)c.Wi);
    a.divWq = FastDiv((uint32_t)std::max(1, c.Wi / 4));
    a.divRIN = FastDiv((uint32_t)a.RIN);
    a.divHW = FastDiv((uint32_t)(c.Hf * c.Wf));
    a.divWf = FastDiv((uint32_t)c.Wf);
    a.swz = knob(KNOB_TILE_ORDER) != 1;
    return true;
}

template <int CPW, bool AVEC, bool XVEC>
int launch_t(const float* x, const float* w, float* y, const SArgs& a, hipStream_t stream)
{
    const void* f = (const void*)conv_f32_small_kernel<CPW, AVEC, XVEC>;
    ensure_lds_limit(f, kLds);
    const int64_t grid = (int64_t)a.co_tiles * a.c.N * a.pt_img;
    hipLaunchKernelGGL((conv_f32_small_kernel<CPW, AVEC, XVEC>), dim3((unsigned)grid), dim3(kNT),
                       a.lds_bytes, stream, x, w, y, a);
    return launch_status();
}

}  // namespace

bool f32_small_applies(const ConvShape& c)
{
    SArgs a;
    int cpw;
    return knob(KNOB_F32_SMALL) >= 0 && plan(c, a, cpw);
}

int launch_conv_f32_small(const float* x, const float* w, float* y, const ConvShape& c,
                          hipStream_t stream)
{
    SArgs a;
    int cpw;
    if (knob(KNOB_F32_SMALL) < 0 || !plan(c, a, cpw)) return -1;
    if ((uintptr_t)x % 4 || (uintptr_t)w % 4 || (uintptr_t)y % 4) return -1;
    // 16-byte loads need 16-byte aligned filter rows and input rows.
    const bool av = a.K % 4 == 0 && (uintptr_t)w % 16 == 0;
    const bool xv = c.Wi % 4 == 0 && (uintptr_t)x % 16 == 0;
    auto go = [&](auto cpw_tag) -> int {
        constexpr int C = decltype(cpw_tag)::value;
        if (av && xv) return launch_t<C, true, true>(x, w, y, a, stream);
        if (av) return launch_t<C, true, false>(x, w, y, a, stream);
        if (xv) return launch_t<C, false, true>(x, w, y, a, stream);
        return launch_t<C, false, false>(x, w, y, a, stream);
    };
    switch (cpw) {
    case 4: return go(std::integral_constant<int, 4>());
    case 8: return go(std::integral_constant<int, 8>());
    case 12: return go(std::integral_constant<int, 12>());
    case 16: return go(std::integral_constant<int, 16>());
    case 20: return go(std::integral_constant<int, 20>());
    case 24: return go(std::integral_constant<int, 24>());
    }
    return -1;
}

}  // namespace im2win
