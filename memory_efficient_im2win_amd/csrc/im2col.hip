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
//    A workgroup writes the rows of up to 32 consecutive pixels of one
//    output row from their input rows, copied into LDS by direct dword
//    loads; shapes whose rows do not fit fall back to 128-byte column tiles
//    of 32 rows, one 16-byte piece per thread.
//  * filter_pad_kernel copies the filters into rows of KP (zero tail).
//  * gemm_tiled_kernel computes y[n][co][p] = sum_k w[co][k] * col[q][k] on
//    the matrix cores with the same instructions and operand layouts as the
//    im2win kernels (v_mfma_f32_32x32x16_f16, v_mfma_f32_32x32x2_f32). A
//    workgroup owns 64 output channels x 256 pixels with 4 waves, or 128
//    channels x 256 pixels with 8 (Co >= 128), each wave 64 x 64 (2 x 2
//    tiles of 32 x 32). A stage is 128 bytes of K of every row of both
//    operands (64 or 128 filter rows + 256 im2col rows = 40 or 48 KB), copied
//    into LDS with buffer_load_dwordx4 ... lds, eight lanes per row (whole
//    128-byte lines of the im2col matrix); two stage buffers (80 KB for the
//    64-channel tile: two workgroups per CU), loads one stage ahead, one
//    barrier per stage. The 16-byte pieces of a row are
//    stored XOR-swizzled by the row's low 3 bits, so the 8 lanes of a read
//    group (8 rows, one piece) hit all banks.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace im2win {

namespace {


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

struct ColVArgs {
    ConvShape c;
    int K, KP, cpr;           // taps, padded row, 16-byte pieces per row
    int ptiles;               // 8-piece (128-byte) column tiles per row
    uint32_t rows;            // N*Ho*Wo
    FastDiv divPlane, divWo, divHW, divWf;
};

// A workgroup writes the 128-byte column tile kt of 32 consecutive rows:
// thread t takes row q0 + t%32 and its 16-byte piece 8*kt + t/32, so the 32
// lanes of a half-wave read one tap of 32 neighbouring windows (nearby
// addresses) and the 8 pieces of every row's 128 bytes are written by one
// workgroup. A piece's first tap is decomposed once; later taps step
// (kw, kh, ci) along.
template <typename T>
__global__ __launch_bounds__(256) void im2col_vec_kernel(const T* __restrict__ x,
                                                         T* __restrict__ col, ColVArgs a)
{
    constexpr int V = 16 / sizeof(T);
    const uint32_t kt = blockIdx.x % (uint32_t)a.ptiles;
    const uint32_t q = (blockIdx.x / (uint32_t)a.ptiles) * 32 + (threadIdx.x & 31);
    const int piece = (int)kt * 8 + (int)(threadIdx.x >> 5);
    if (q >= a.rows || piece >= a.cpr) return;
    const int k0 = piece * V;
    const uint32_t n = a.divPlane.div(q);
    const int pix = (int)(q - n * (uint32_t)(a.c.Ho * a.c.Wo));
    const int ho = (int)a.divWo.div((uint32_t)pix), wo = pix - ho * a.c.Wo;
    const int ci = (int)a.divHW.div((uint32_t)k0);
    const int r = k0 - ci * a.c.Hf * a.c.Wf;
    int kh = (int)a.divWf.div((uint32_t)r), kw = r - kh * a.c.Wf;
    // Offsets within the image (below 2^31 elements): the window corner,
    // then tap (ci, kh, kw) relative to it, stepped along the taps.
    const T* xw = x + (int64_t)n * a.c.Ci * a.c.Hi * a.c.Wi +
                  ((int64_t)ho * a.c.sh) * a.c.Wi + (int64_t)wo * a.c.sw;
    int off = (ci * a.c.Hi + kh) * a.c.Wi + kw;
    const int row_skip = a.c.Wi - a.c.Wf, chan_skip = (a.c.Hi - a.c.Hf) * a.c.Wi;
    T v[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        v[u] = k0 + u < a.K ? xw[off] : T(0);
        ++off;
        if (++kw == a.c.Wf) {
            kw = 0;
            off += row_skip;
            if (++kh == a.c.Hf) {
                kh = 0;
                off += chan_skip;
            }
        }
    }
    uint4 o;
    __builtin_memcpy(&o, v, 16);
    reinterpret_cast<uint4*>(col)[(int64_t)q * a.cpr + piece] = o;
}

// A direct global-to-LDS load of one dword per lane: lane l's dword at
// voff in r lands at LDS byte lds + 4*l (zero for an offset past r).
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff)
{
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(voff), "s"(r)
        : "memory");
}

constexpr int64_t kColLds = 40 * 1024;
constexpr uint32_t kColMiss = 0xFFFFFFF0u;   // a load offset past any x buffer

struct ColRArgs {
    ConvShape c;
    int K, KP, cpr;           // taps, padded row, 16-byte pieces per row
    int cols;                 // LDS row pitch: (seg-1)*sw + Wf rounded up to whole dwords
    int seg;                  // pixels per row segment
    int wtiles;               // segments per output row
    int units;                // dwords per LDS row (cols * sizeof(T) / 4)
    int64_t xbytes;           // bytes of x
    FastDiv divCpr, divHW, divWf, divUnits;
};

// A workgroup writes the im2col rows of a segment of seg (32, 16 or 8)
// consecutive pixels of one output row (npx <= seg rows, contiguous in
// col): it first copies the input rows
// their windows cover, every channel, columns c0 .. c0 + cols - 1, into LDS
// ([ci][kh][col]); then consecutive threads build consecutive 16-byte
// pieces of those rows from LDS, so every store instruction writes 1 KB of
// consecutive bytes.
template <typename T>
__global__ __launch_bounds__(256) void im2col_rows_kernel(const T* __restrict__ x,
                                                          T* __restrict__ col, ColRArgs a)
{
    constexpr int V = 16 / sizeof(T);
    extern __shared__ __align__(16) unsigned char smem_c[];
    T* Xs = reinterpret_cast<T*>(smem_c);
    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Hf = a.c.Hf, Wf = a.c.Wf;
    const int Ho = a.c.Ho, Wo = a.c.Wo, sw = a.c.sw;
    const int wt = (int)(blockIdx.x % (uint32_t)a.wtiles);
    const int rest = (int)(blockIdx.x / (uint32_t)a.wtiles);
    const int ho = rest % Ho, n = rest / Ho;
    const int w0 = wt * a.seg;
    const int npx = min(a.seg, Wo - w0);
    const int c0 = w0 * sw;
    const int ncol = min(a.cols, Wi - c0);

    // Input rows (ci, ho*sh + kh), columns c0 .. c0 + ncol - 1, copied a
    // dword at a time (Wi*sizeof(T) and c0*sizeof(T) are multiples of 4)
    // straight into LDS by direct loads, all in flight at once: wave v takes
    // the 64-dword pieces v, v+4, ... of the rows. LDS row r = ci*Hf + kh;
    // dwords past a row's input columns, and past the last row up to the
    // whole piece, load zeros (offsets past the buffer).
    const uint32_t lbase =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem_c;
    const T* xb = x + (((int64_t)n * Ci) * Hi + (int64_t)ho * a.c.sh) * Wi + c0;
    const int64_t xoff = (int64_t)(xb - x) * (int64_t)sizeof(T);
    const __amdgpu_buffer_rsrc_t rx =
        raw_rsrc(xb, (uint32_t)(a.xbytes - xoff < (int64_t)kColMiss ? a.xbytes - xoff
                                                                   : (int64_t)kColMiss));
    constexpr int EPU = 4 / sizeof(T);
    const int uw = (ncol + EPU - 1) / EPU;      // dwords of a row to copy
    const int total_u = Ci * Hf * a.units;
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    for (int pc = wave; pc * 64 < total_u; pc += 4) {
        const int e = pc * 64 + lane;
        const int r = (int)a.divUnits.div((uint32_t)e), j = e - r * a.units;
        const int ci = r / Hf, kh = r - ci * Hf;
        const uint32_t v = e < total_u && j < uw
                               ? (uint32_t)((((int64_t)ci * Hi + kh) * Wi) * (int64_t)sizeof(T)) + 4u * j
                               : kColMiss;
        lds_dma4(rx, lbase + (uint32_t)pc * 256u, v);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Pieces of rows q0 .. q0 + npx - 1: piece e = (pixel e / cpr, piece e % cpr).
    T* out = col + (((int64_t)n * Ho + ho) * Wo + w0) * a.KP;
    const int total = npx * a.cpr;
    for (int e = threadIdx.x; e < total; e += 256) {
        const int qi = (int)a.divCpr.div((uint32_t)e);
        const int pc = e - qi * a.cpr;
        const int k0 = pc * V;
        const int ci = (int)a.divHW.div((uint32_t)k0);
        const int rr = k0 - ci * Hf * Wf;
        const int kh = (int)a.divWf.div((uint32_t)rr);
        int kw = rr - kh * Wf;
        // LDS row index ci*Hf + kh steps by one when kw wraps.
        int off = (ci * Hf + kh) * a.cols + qi * sw + kw;
        T v[V];
#pragma unroll
        for (int u = 0; u < V; ++u) {
            v[u] = k0 + u < a.K ? Xs[off] : T(0);
            ++off;
            if (++kw == Wf) {
                kw = 0;
                off += a.cols - Wf;
            }
        }
        uint4 o;
        __builtin_memcpy(&o, v, 16);
        reinterpret_cast<uint4*>(out)[e] = o;
    }
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

// Tiles of TM output channels (64: 4 waves; 128: 8 waves, two 64-channel
// halves) by kTN pixels.
constexpr int kTN = 256;                   // pixels per tile
constexpr int kSB = 128;                   // bytes of K per row and stage
constexpr int kTBufs = 2;                  // stage buffers: loads one stage ahead
template <int TM> struct TileCfg {
    static constexpr int kNW = TM / 16;                         // waves
    static constexpr int kStage = (TM + kTN) * kSB;             // 40 or 48 KB
    static constexpr int kSlots = kStage / 1024 / kNW;          // 1-KB loads per wave and stage
    static constexpr int kLds = kTBufs * kStage;               // 80 or 96 KB
    static_assert(kStage % (1024 * kNW) == 0, "whole slots per wave");
};
constexpr uint32_t kTMiss = 0xFFFFFFF0u;

// Byte offset of row `row`'s 16-byte piece c in a stage region (pieces
// XOR-swizzled by the row's low 3 bits).
__device__ __forceinline__ uint32_t tpos(int row, int c) { return row * kSB + ((c ^ (row & 7)) << 4); }

template <bool F16, int TM>
__global__ __launch_bounds__(TM * 4) void gemm_tiled_kernel(const void* __restrict__ colv,
                                                            const void* __restrict__ wv,
                                                            float* __restrict__ y, GemmArgs a)
{
    constexpr int E = F16 ? 2 : 4;
    constexpr int kTM = TM, kNW = TileCfg<TM>::kNW, kTStage = TileCfg<TM>::kStage;
    constexpr int kTSlots = TileCfg<TM>::kSlots;
    extern __shared__ __align__(16) unsigned char smem[];
    const uint32_t lbase =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    const int lane = threadIdx.x & 63, hl = lane >> 5, l32 = lane & 31;
    const int wave = uniform(threadIdx.x >> 6);
    const int wc = wave >> 2, wp = wave & 3;   // 64-channel half, 64-pixel quarter
    const int co_tiles = (a.Co + kTM - 1) / kTM;
    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x, true);
    const int co0 = (int)(bid % co_tiles) * kTM;
    const int64_t q0 = (bid / co_tiles) * kTN;

    // Load slots: slot m of a stage is LDS kilobyte m = rows 8m .. 8m+7 of
    // the stage region (filter rows 0 .. TM-1 first, then im2col rows
    // 0-255); wave v issues slots v, v+NW, ... Lane l loads row 8m + l/8,
    // its piece (l%8) ^ (l/8) to land at piece l%8 of the swizzle.
    uint32_t voff[kTSlots];
    bool isw[kTSlots];
#pragma unroll
    for (int i = 0; i < kTSlots; ++i) {
        const int m = wave + kNW * i;
        const int row = 8 * m + (lane >> 3);
        const int pc = (lane & 7) ^ (lane >> 3);
        uint32_t v = kTMiss;
        isw[i] = m < kTM / 8;
        if (isw[i]) {
            const int co = co0 + row;
            if (co < a.Co) v = (uint32_t)((int64_t)co * a.KP * E) + pc * 16;
        } else {
            const int64_t q = q0 + (row - kTM);
            if (q < a.rows) {
                int64_t r = q * a.KP;
                if (a.win_rows) {
                    const int64_t n = q / a.P;
                    const int pix = (int)(q - n * a.P);
                    const int ho = pix / a.Wo, wo = pix - ho * a.Wo;
                    r = ((n * a.Ho + ho) * a.Wi + (int64_t)wo * a.sw) * a.HfC;
                }
                const uint64_t b = (uint64_t)r * E + pc * 16;
                if (b < kTMiss) v = (uint32_t)b;
            }
        }
        voff[i] = v;
    }
    const int nbytes = a.KP * E;                // bytes of K per row
    const int NS = (nbytes + kSB - 1) / kSB;    // stages
    auto issue = [&](int s, int sb) {
        const uint32_t ko = (uint32_t)s * kSB;
        const __amdgpu_buffer_rsrc_t rw =
            raw_rsrc((const unsigned char*)wv + ko, (uint32_t)(a.wbytes - ko));
        const __amdgpu_buffer_rsrc_t rc =
            raw_rsrc((const unsigned char*)colv + ko, (uint32_t)(a.colbytes - ko));
        const uint32_t base = lbase + (uint32_t)sb * kTStage;
#pragma unroll
        for (int i = 0; i < kTSlots; ++i)
            lds_dma16(isw[i] ? rw : rc, base + (uint32_t)(wave + kNW * i) * 1024, voff[i]);
    };

    floatx16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // A: filter rows 64*wc + i*32 + l32; B: im2col rows kTM + 64*wp + 32*j + l32.
    // Slice t (32 bytes of K) of a stage: lane half hl reads piece 2t + hl.
    auto slice = [&](const unsigned char* S, int t) {
        uint4 A[2], B[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            __builtin_memcpy(&A[i], S + tpos(64 * wc + i * 32 + l32, 2 * t + hl), 16);
            __builtin_memcpy(&B[i], S + tpos(kTM + 64 * wp + 32 * i + l32, 2 * t + hl), 16);
        }
        if constexpr (F16) {
            half8_t ah[2], bh[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                __builtin_memcpy(&ah[i], &A[i], 16);
                __builtin_memcpy(&bh[i], &B[i], 16);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bh[j], acc[i][j], 0, 0, 0);
        } else {
            // Lane half hl holds K values k0 + 4*hl + u for step u.
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float af[2], bf[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    uint32_t ua, ub;
                    __builtin_memcpy(&ua, reinterpret_cast<const uint32_t*>(&A[i]) + u, 4);
                    __builtin_memcpy(&ub, reinterpret_cast<const uint32_t*>(&B[i]) + u, 4);
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

    issue(0, 0);
    for (int s = 0; s < NS; ++s) {
        wait_vm<0>();         // this wave's loads of stage s have landed
        __syncthreads();      // every wave's; and stage s-1's buffer is free
        if (s + 1 < NS) issue(s + 1, (s + 1) % kTBufs);
        const unsigned char* S = smem + (size_t)(s % kTBufs) * kTStage;
        const int ns = min(kSB, nbytes - s * kSB) / 32;   // 32-byte slices in this stage
        if (ns == kSB / 32) {
#pragma unroll
            for (int t = 0; t < kSB / 32; ++t) slice(S, t);
        } else {
            for (int t = 0; t < ns; ++t) slice(S, t);
        }
    }
    wait_vm<0>();

    // Output: lane holds pixel l32 of each block and channels
    // 8*(r/4) + 4*hl + r%4 of each 32-channel block.
    const __amdgpu_buffer_rsrc_t ry = gbuf(y, a.ybytes);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t q = q0 + 64 * wp + j * 32 + l32;
        if (q >= a.rows) continue;
        const int64_t n = q / a.P;
        const int p = (int)(q - n * a.P);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = co0 + 64 * wc + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
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
    // 128-channel tiles (8 waves, two per SIMD) when the channels fill a
    // whole one and the tiles still cover the 256 CUs: half the passes over
    // the matrix (cv5 fp16: 217 against 270 us per im2col call). With 96
    // channels either tile wastes a quarter, and the 64-channel one ran
    // faster; a small batch (cv5 fp32, N = 1: 4 tiles of 128) needs the
    // 64-channel tiles' parallelism.
    const int64_t ptiles = (g.rows + kTN - 1) / kTN;
    const int TM = Co >= 128 && ptiles * ((Co + 127) / 128) >= 256 ? 128 : 64;
    const int64_t blocks = ptiles * ((Co + TM - 1) / TM);
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    auto go = [&](auto kern, int tm, int lds) {
        ensure_lds_limit((const void*)kern, lds);
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(tm * 4), lds, stream, b, a, y, g);
    };
    if (elem == 2) {
        if (TM == 128) go(gemm_tiled_kernel<true, 128>, 128, TileCfg<128>::kLds);
        else go(gemm_tiled_kernel<true, 64>, 64, TileCfg<64>::kLds);
    } else {
        if (TM == 128) go(gemm_tiled_kernel<false, 128>, 128, TileCfg<128>::kLds);
        else go(gemm_tiled_kernel<false, 64>, 64, TileCfg<64>::kLds);
    }
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
    const int cpr = a.KP * elem / 16;   // KP*elem is a multiple of 32 bytes
    {
        // Row-segment kernel when a segment's input rows fit in 80 KB of LDS.
        ColRArgs r;
        r.c = c;
        r.K = a.K;
        r.KP = a.KP;
        r.cpr = cpr;
        const int epu = 4 / elem;
        // The longest segment (32, 16 or 8 pixels) whose rows take at most
        // 40 KB of LDS, so that four workgroups share a CU.
        int64_t lds = 0;
        for (int seg : {32, 16, 8}) {
            r.seg = seg;
            r.cols = (std::min((seg - 1) * c.sw + c.Wf, c.Wi) + epu - 1) / epu * epu;
            // Whole 256-byte pieces: the direct loads fill the last one.
            lds = ((int64_t)c.Ci * c.Hf * r.cols * elem + 255) / 256 * 256;
            if (lds <= kColLds) break;
        }
        r.units = r.cols / epu;
        r.wtiles = (c.Wo + r.seg - 1) / r.seg;
        const int64_t rblocks = (int64_t)c.N * c.Ho * r.wtiles;
        if (lds <= 80 * 1024 && rblocks < 0x7fffffff && (uintptr_t)col % 16 == 0 &&
            c.Wi % epu == 0 && (uintptr_t)x % 4 == 0) {
            r.xbytes = (int64_t)c.N * c.Ci * c.Hi * c.Wi * elem;
            r.divUnits = FastDiv((uint32_t)r.units);
            r.divCpr = FastDiv((uint32_t)cpr);
            r.divHW = FastDiv((uint32_t)(c.Hf * c.Wf));
            r.divWf = FastDiv((uint32_t)c.Wf);
            if (elem == 2) {
                ensure_lds_limit((const void*)im2col_rows_kernel<uint16_t>, 80 * 1024);
                hipLaunchKernelGGL(im2col_rows_kernel<uint16_t>, dim3((unsigned)rblocks), dim3(256),
                                   (unsigned)lds, stream, (const uint16_t*)x, (uint16_t*)col, r);
            } else {
                ensure_lds_limit((const void*)im2col_rows_kernel<uint32_t>, 80 * 1024);
                hipLaunchKernelGGL(im2col_rows_kernel<uint32_t>, dim3((unsigned)rblocks), dim3(256),
                                   (unsigned)lds, stream, (const uint32_t*)x, (uint32_t*)col, r);
            }
            return launch_status();
        }
    }
    const int ptiles = (cpr + 7) / 8;
    const int64_t vblocks = (a.rows + 31) / 32 * ptiles;
    if (a.rows < 0x7fffffff && vblocks < 0x7fffffff && (uintptr_t)col % 16 == 0) {
        ColVArgs v;
        v.c = c;
        v.K = a.K;
        v.KP = a.KP;
        v.cpr = cpr;
        v.ptiles = ptiles;
        v.rows = (uint32_t)a.rows;
        v.divPlane = FastDiv((uint32_t)(c.Ho * c.Wo));
        v.divWo = FastDiv((uint32_t)c.Wo);
        v.divHW = FastDiv((uint32_t)(c.Hf * c.Wf));
        v.divWf = FastDiv((uint32_t)c.Wf);
        if (elem == 2)
            hipLaunchKernelGGL(im2col_vec_kernel<uint16_t>, dim3((unsigned)vblocks), dim3(256), 0,
                               stream, (const uint16_t*)x, (uint16_t*)col, v);
        else
            hipLaunchKernelGGL(im2col_vec_kernel<uint32_t>, dim3((unsigned)vblocks), dim3(256), 0,
                               stream, (const uint32_t*)x, (uint32_t*)col, v);
        return launch_status();
    }
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

int launch_nhwc_gemm(const void* ws, const void* wr, float* y, const ConvShape& c, int elem,
                     hipStream_t stream)
{
    GemmArgs g{};
    g.Co = c.Co;
    g.HfC = nhwc_pitch(c, elem);   // runs padded to a multiple of 32 bytes
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
