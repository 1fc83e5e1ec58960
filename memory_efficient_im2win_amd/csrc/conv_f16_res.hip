// fp16 im2win convolution on the CDNA4 matrix cores with a tile's input
// resident in LDS for the whole reduction and the filter streamed from the L2
// cache into registers (fp32 accumulate; prepacked filter).
//
// The half-precision path of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract: half
// precision multiply-accumulate on matrix hardware; Table I, cv5: 256 filters
// of 96 x 5 x 5 over 24 x 24 inputs), on the im2win rows of "Im2win: Memory
// Efficient Convolution On SIMD Architectures" (Abstract): the inputs of one
// window row are one contiguous run of an input row, so a tile that owns R
// whole output rows of one image needs exactly the (R-1)*sh + Hf input rows
// behind them, and those rows hold every window of the tile.
//
//  * A workgroup owns 256 output channels x R output rows of one image
//    (cv5: R = 10, 200 pixels; two tiles per image, 256 tiles at N = 128,
//    one per CU). It copies its input rows of every channel into LDS once,
//    channel-interleaved (one 16-byte entry = 8 channels of one input column,
//    rows Wi entries apart; cv5: 12 octets x 14 rows x 24 columns = 64.5 KB),
//    and they stay there for the whole reduction: no stages, no barrier
//    after the copy.
//  * GEMM view: rows = the tile's pixels, columns = output channels (NHWC:
//    the other way round, so a lane holds 4 consecutive channels of one
//    output pixel), K = (channel quad q of 32, tap (kh, kw), channel). A K
//    step of 32 is one tap of 32 channels; lanes 16g..16g+15 take octet
//    4q + g, so every lane's 8-element slice is one aligned 16-byte read:
//    from LDS for the pixels, from the prepacked filter for the channels. No
//    tap is padded.
//  * NHWC tensors (the fused NHWC call): the 8 channels of an input pixel
//    are 16 contiguous bytes of x, so the tile's rows are copied into LDS as
//    they lie, pixel-major with an odd number of entries per pixel.
//  * 8 waves, two per SIMD. Waves w and w + 4 hold channels 64(w % 4) ..
//    +63 (4 blocks of 16) and split the tile's pixel blocks of 16 (cv5: 13
//    blocks as 7 + 6; 16 x 16 accumulators, 112 registers). Per K step a
//    wave reads one fragment per pixel block from LDS, each feeding 4 MFMAs,
//    and loads its 4 filter fragments into registers two steps ahead (the
//    whole filter, 1.2 MB on cv5, stays in every XCD's L2). The second wave
//    of a SIMD covers the first one's waits (1.06x over 4 waves of 128
//    channels, which read half the LDS bytes).
//  * The tile's input copy at the start and its 205 KB of output stores at
//    the end are not overlapped with MFMAs: the 256 tiles of cv5 run in one
//    round (cv5: 61-63 us, against 27-30 us of MFMA issue at the measured
//    clock).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "knobs.hpp"

namespace im2win {

namespace {

constexpr int kResCo = 256;               // output channels per tile (4 groups of 64)
constexpr int kResLds = 160 * 1024;
constexpr uint32_t kMissR = 0xFFFFFFF0u;  // vector offset past every accepted buffer

struct ResArgs {
    ConvShape c;
    int R;            // output rows per tile
    int tpi;          // tiles per image: ceil(Ho / R)
    int co_tiles;     // Co / 256
    int Rin;          // input rows of a tile: (R - 1) * sh + Hf
    int Q;            // channel quads of 32
    int OS;           // LDS entries per octet: Rin * Wi
    int ppo;          // column pairs per octet: OS / 2
    int OCTP;         // NHWC: LDS entries per staged pixel, 4(Q + 1) + 1 (odd: no bank conflicts)
    int tasks;        // copy tasks: channel octets x ppo pairs
    int HW, HWp, Copad, S;   // taps; prepacked layout; K steps Q * HW
    int Spad;         // K steps run: S rounded up to a multiple of 3
    uint32_t lds_bytes;
    uint32_t xbytes, ybytes, wbytes;
    FastDiv divCoT, divTpi, divWo, divWf, divHW, divPpo, divOCTP;
    bool swz;         // XCD-grouped tile order
};

template <int K>
struct IC {
    static constexpr int value = K;
};

// acc += a * b on the matrix cores (v_mfma_f32_16x16x32_f16, a: 16 rows x 32
// of K, b: 32 of K x 16 columns), with the accumulator tied to one AGPR
// quadruple for input and output. Through the builtin, the register
// allocator gives each of the many 4-register accumulators of this kernel
// a new place at every MFMA and copies them around the K loop (hundreds of
// AGPR moves per step). Hazards: consecutive MFMAs on one accumulator are
// exactly overlapped (no wait states), and the accumulators are read only
// after mfma_drain().
__device__ __forceinline__ void mfma16(floatx4_t& acc, const half8_t& a, const half8_t& b)
{
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states before any instruction reads an accumulator an MFMA wrote
// (more than the 16-pass MFMA's requirement).
__device__ __forceinline__ void mfma_drain()
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// 16 bytes of an accumulator stored at byte voff of buffer r (a vector
// store that reads the AGPRs directly; out-of-range offsets are dropped).
__device__ __forceinline__ void store16(const floatx4_t& v, __amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen" ::"a"(v), "v"(voff), "s"(r) : "memory");
}

// The reduction and the stores of one wave: channels co_base .. +63 (4
// blocks of 16) x pixel blocks jb .. jb+NBW-1 of the tile, the input rows in
// LDS (smem), the filter read from wpk.
template <int NBW, int NCB, bool NHWC>
__device__ __forceinline__ void res_compute(const unsigned char* smem, const uint4* __restrict__ wpk,
                                            float* __restrict__ y, const ResArgs& a, int co_base,
                                            int jb, int P, uint32_t n, int ho0, int lane)
{
    const int Wi = a.c.Wi, Co = a.c.Co, sh = a.c.sh, sw = a.c.sw;
    const int Ho = a.c.Ho, Wo = a.c.Wo, Wf = a.c.Wf;
    const int g = lane >> 4, c16 = lane & 15;

    // LDS byte address of tap (0, 0) of this lane's pixel in each block, in
    // octet g of quad 0 (pixels past the tile read pixel 0; never stored).
    uint32_t bb[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        int p = 16 * (jb + j) + c16;
        if (p >= P) p = 0;
        const int r = (int)a.divWo.div((uint32_t)p);
        const int wo = p - r * Wo;
        bb[j] = NHWC ? (uint32_t)(((r * sh * Wi + wo * sw) * a.OCTP + g) * 16)
                     : (uint32_t)((g * a.OS + r * sh * Wi + wo * sw) * 16);
    }
    // This lane's filter entry in K step (q, tap): ((4q + g) * HWp + tap) *
    // Copad + co_base + 16b + c16; the uniform part goes into the resource's
    // base, octets past the filter (and every step from S on) read zeros.
    const uint32_t aoff = (uint32_t)((g * a.HWp * a.Copad + c16) * 16);

    // Each accumulator starts from a zero the compiler cannot share between
    // them: a shared zero constant makes it copy every 4-register
    // accumulator around the K loop instead of keeping it in place.
    floatx4_t acc[NBW][NCB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < NCB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float z;
                asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(z));
                acc[j][b][r] = z;
            }

    half8_t af[3][NCB];   // filter fragments: ring slot (K step mod 3) x channel block
    half8_t bf[NBW];     // pixel fragments of the current step, replaced block by block

    auto load_a = [&](int slot, int s) {
        const int q = (int)a.divHW.div((uint32_t)s);
        const int tap = s - q * a.HW;
        const int64_t ent = ((int64_t)4 * q * a.HWp + tap) * a.Copad + co_base;
        const uint32_t left = ent * 16 < (int64_t)a.wbytes ? a.wbytes - (uint32_t)(ent * 16) : 0u;
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(left ? wpk + ent : wpk, left);
#pragma unroll
        for (int b = 0; b < NCB; ++b) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(aoff + b * 256), 0, 0);
            __builtin_memcpy(&af[slot][b], &v, 16);
        }
    };
    auto b_off = [&](int s) {
        const int q = (int)a.divHW.div((uint32_t)s);
        const int tap = s - q * a.HW;
        const int kh = (int)a.divWf.div((uint32_t)tap);
        const int kw = tap - kh * Wf;
        return NHWC ? (uint32_t)(((kh * Wi + kw) * a.OCTP + 4 * q) * 16)
                    : (uint32_t)((4 * q * a.OS + kh * Wi + kw) * 16);
    };
    // K step s: the filter of step s+2 is loaded (a ring of 3 steps); then
    // block by block, the 4 MFMAs of step s on pixel block j, and block j of
    // step s+1 read into its place (NBW-1 blocks of MFMAs ahead of its use).
    // The loop runs Spad steps, a multiple of 3, with no tail: steps from S
    // on read zero filter fragments and the zero octets and add exact zeros
    // (one loop whose steps all issue the same loads keeps the compiler's
    // load counts exact and the accumulators in place).
    auto body = [&](auto K, int s) {
        constexpr int k = decltype(K)::value;
        load_a((k + 2) % 3, s + 2);
        const uint32_t o = b_off(s + 1);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
#pragma unroll
            for (int b = 0; b < NCB; ++b) {
                if (NHWC)
                    mfma16(acc[j][b], af[k][b], bf[j]);   // rows: channels
                else
                    mfma16(acc[j][b], bf[j], af[k][b]);   // rows: pixels
            }
            bf[j] = *reinterpret_cast<const half8_t*>(smem + bb[j] + o);
        }
    };

    load_a(0, 0);
    load_a(1, 1);
#pragma unroll
    for (int j = 0; j < NBW; ++j) bf[j] = *reinterpret_cast<const half8_t*>(smem + bb[j] + b_off(0));
    // Spad >= 3: a loop that always runs, so no path around it reaches the
    // stores with the accumulators in other registers.
    int s = 0;
#pragma nounroll
    do {
        body(IC<0>{}, s);
        body(IC<1>{}, s + 1);
        body(IC<2>{}, s + 2);
        s += 3;
    } while (s < a.Spad);

    mfma_drain();

    const __amdgpu_buffer_rsrc_t ry = raw_rsrc(y, a.ybytes);
    if (NHWC) {
        // Lane (g, c16) of block (j, b) holds channels co_base + 16b + 4g ..
        // +3 of pixel 16j + c16: 16 contiguous bytes of y (N x Ho x Wo x Co).
        const int64_t row0 = ((int64_t)n * Ho + ho0) * Wo;
#pragma unroll
        for (int b = 0; b < NCB; ++b) {
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const int p = 16 * (jb + j) + c16;
                const uint32_t off =
                    (uint32_t)(((row0 + p) * Co + co_base + 16 * b + 4 * g) * 4);
                store16(acc[j][b], ry, p < P ? off : kMissR);
            }
        }
        return;
    }
    // Lane (g, c16) of block (j, b) holds pixels 16j + 4g .. +3 of channel
    // co_base + 16b + c16 (4 consecutive floats, 16-byte aligned as Wo % 4
    // == 0): one 16-byte store straight from the accumulator registers,
    // ordered after the wait states (the stores are statements of the same
    // kind as the MFMAs, which keep their order); pixels past the tile get
    // an offset out of range and are dropped.
    const int64_t plane = (int64_t)Ho * Wo;
#pragma unroll
    for (int b = 0; b < NCB; ++b) {
        const int co = co_base + 16 * b + c16;
        const uint32_t base = (uint32_t)((((int64_t)n * Co + co) * plane + (int64_t)ho0 * Wo) * 4);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int p0 = 16 * (jb + j) + 4 * g;
            store16(acc[j][b], ry, p0 < P ? base + p0 * 4 : kMissR);
        }
    }
}

// NB pixel blocks per tile; NCB channel blocks per wave: 2 * 256 / (16 NCB)
// waves (NCB = 8: 4 waves, one per SIMD; NCB = 4: 8 waves, two per SIMD).
// NHWC: x is N x Hi x Wi x Ci and y N x Ho x Wo x Co.
template <int NB, int NCB, bool NHWC>
__global__ __launch_bounds__(128 * kResCo / (16 * NCB)) void conv_f16_res_kernel(const uint16_t* __restrict__ x,
                                                             const uint4* __restrict__ wpk,
                                                             float* __restrict__ y, ResArgs a)
{
    constexpr int NT = 128 * kResCo / (16 * NCB);
    extern __shared__ __align__(16) unsigned char smem[];
    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, sh = a.c.sh, Ho = a.c.Ho, Wo = a.c.Wo;

    // Tile: channel tile fastest, then the row tiles of an image, then images.
    const uint32_t bid = (uint32_t)xcd_tile(blockIdx.x, gridDim.x, a.swz);
    const uint32_t pt = a.divCoT.div(bid);
    const int co_t = (int)(bid - pt * (uint32_t)a.co_tiles);
    const uint32_t n = a.divTpi.div(pt);
    const int tr = (int)(pt - n * (uint32_t)a.tpi);
    const int ho0 = tr * a.R;
    const int P = min(a.R, Ho - ho0) * Wo;   // pixels of the tile
    const int ih0 = ho0 * sh;
    const int tid = threadIdx.x;

    if (NHWC) {
        // NHWC: the tile's input rows are one contiguous block of x, whose 16
        // bytes at (pixel, octet o) are exactly the entry of those 8 channels;
        // entry e = pixel * OCTP + o takes them for o < Ci/8 and zeros
        // otherwise (the octets padding the last quad, the 4 zero octets the
        // K steps past S read, and the spare entry that makes OCTP odd).
        // Consecutive threads write consecutive entries.
        const __amdgpu_buffer_rsrc_t rx = raw_rsrc(x, a.xbytes);
        const int octs = Ci >> 3;
        const int pix = min(a.Rin, Hi - ih0) * Wi;   // staged pixels that exist
        const int64_t base = ((int64_t)n * Hi + ih0) * Wi;
        const int total = a.Rin * Wi * a.OCTP;
        uint4* L = reinterpret_cast<uint4*>(smem);
        constexpr int U = 4;
        for (int e0 = 0; e0 < total; e0 += U * NT) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = e0 + u * NT + tid;
                const int px = (int)a.divOCTP.div((uint32_t)e);
                const int o = e - px * a.OCTP;
                const uint32_t off = e < total && o < octs && px < pix
                                         ? (uint32_t)(((base + px) * Ci + 8 * o) * 2)
                                         : kMissR;
                const auto r = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
                v[u] = make_uint4(r[0], r[1], r[2], r[3]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = e0 + u * NT + tid;
                if (e < total) L[e] = v[u];
            }
        }
    } else
    // Copy the tile's input rows into LDS. Task (octet o, column pair m) of
    // the octets that hold channels: one dword (columns 2m and 2m+1 of the
    // staged rows, which are one contiguous run per channel) from each of
    // its 8 channel planes, split into the two entries 2m and 2m+1; rows
    // past Hi and channels past Ci read zeros. Consecutive threads take
    // consecutive pairs, so the loads of a wave are 256 contiguous bytes of
    // a plane and its LDS writes 32 bytes apart (no bank conflicts). The
    // octets past the last channel octet, up to and including the 4 zero
    // octets that the K steps past S read, are written as zeros.
    {
        const __amdgpu_buffer_rsrc_t rx = raw_rsrc(x, a.xbytes);
        const int64_t img = (int64_t)n * Ci;
        const int pairs = (min(a.Rin, Hi - ih0) * Wi) >> 1;   // pairs of existing rows
        uint4* L = reinterpret_cast<uint4*>(smem);
        constexpr int U = 4;
        for (int t0 = 0; t0 < a.tasks; t0 += U * NT) {
            uint32_t d[U][8];
            int dst[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int t = t0 + u * NT + tid;
                const int o = (int)a.divPpo.div((uint32_t)t);
                const int m = t - o * a.ppo;
                dst[u] = t < a.tasks ? o * a.OS + 2 * m : -1;
                const bool rowok = t < a.tasks && m < pairs;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int ch = 8 * o + k;
                    const uint32_t off =
                        rowok && ch < Ci
                            ? (uint32_t)((((img + ch) * Hi + ih0) * Wi + 2 * m) * 2)
                            : kMissR;
                    d[u][k] = __builtin_amdgcn_raw_buffer_load_b32(rx, (int)off, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (dst[u] < 0) continue;
                uint4 lo, hi;
                lo.x = (d[u][0] & 0xffffu) | (d[u][1] << 16);
                lo.y = (d[u][2] & 0xffffu) | (d[u][3] << 16);
                lo.z = (d[u][4] & 0xffffu) | (d[u][5] << 16);
                lo.w = (d[u][6] & 0xffffu) | (d[u][7] << 16);
                hi.x = (d[u][0] >> 16) | (d[u][1] & 0xffff0000u);
                hi.y = (d[u][2] >> 16) | (d[u][3] & 0xffff0000u);
                hi.z = (d[u][4] >> 16) | (d[u][5] & 0xffff0000u);
                hi.w = (d[u][6] >> 16) | (d[u][7] & 0xffff0000u);
                L[dst[u]] = lo;
                L[dst[u] + 1] = hi;
            }
        }
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        for (int e = a.tasks * 2 + tid; e < (int)(a.lds_bytes / 16); e += NT) L[e] = z;
    }

    __syncthreads();   // the input rows

    // Channel groups of 16 NCB channels; two waves per group split the pixel
    // blocks: the first takes blocks 0 .. ceil(NB/2)-1, the second the rest.
    constexpr int G = kResCo / (16 * NCB);
    const int wave = uniform(tid >> 6);
    const int co_base = co_t * kResCo + (wave % G) * 16 * NCB;
    if (wave < G)
        res_compute<(NB + 1) / 2, NCB, NHWC>(smem, wpk, y, a, co_base, 0, P, n, ho0, tid & 63);
    else
        res_compute<NB / 2, NCB, NHWC>(smem, wpk, y, a, co_base, (NB + 1) / 2, P, n, ho0,
                                       tid & 63);
}

constexpr int kResNBs[] = {8, 10, 13};

// Plans a launch; false outside the envelope: Co a multiple of 256, at least
// 4 taps (the steps read past S stay within the zero octets), channel quads
// at most 1/8 padding, a tile's input rows and 4 zero octets within LDS,
// tensors addressable with 32-bit buffer offsets; NCHW: Wi a multiple of 8
// (whole 16-byte chunks per row) and Wo of 4 (whole 16-byte output stores);
// NHWC: Ci a multiple of 8 (whole 16-byte chunks per pixel). R is chosen for
// the fewest rounds of tiles over the CUs times the pixel blocks per tile.
bool plan(const ConvShape& c, ResArgs& a, size_t copad_mult, bool nhwc)
{
    if (knob(KNOB_F16_RES) < 0) return false;
    if (c.Co % kResCo != 0 || c.Hf * c.Wf < 4) return false;
    if (nhwc ? c.Ci % 8 != 0 : (c.Wi % 8 != 0 || c.Wo % 4 != 0)) return false;
    const int oct = ceil_div(c.Ci, 8);
    const int Q = ceil_div(oct, 4);
    if ((32 * Q - c.Ci) * 8 > 32 * Q) return false;
    a.c = c;
    a.Q = Q;
    a.OCTP = 4 * (Q + 1) + 1;
    a.HW = c.Hf * c.Wf;
    a.HWp = (a.HW + 1) & ~1;
    a.Copad = (int)(ceil_div(c.Co, (int)copad_mult) * (int)copad_mult);
    a.co_tiles = c.Co / kResCo;
    a.S = Q * a.HW;
    a.Spad = (a.S + 2) / 3 * 3;
    const int cus = 256;
    const int per_pixel = nhwc ? a.OCTP : 4 * (Q + 1);   // LDS entries per staged pixel
    int best_R = 0;
    double best = 0;
    for (int R = 1; R <= c.Ho; ++R) {
        const int need = ceil_div(R * c.Wo, 16);
        int nb = 0;
        for (int v : kResNBs)
            if (v >= need) {
                nb = v;
                break;
            }
        if (nb == 0) break;
        const int Rin = (R - 1) * c.sh + c.Hf;
        if ((int64_t)per_pixel * Rin * c.Wi * 16 > kResLds) break;
        const int64_t tiles = (int64_t)c.N * ceil_div(c.Ho, R) * a.co_tiles;
        const double cost = (double)((tiles + cus - 1) / cus) * nb;
        if (best_R == 0 || cost <= best) {
            best = cost;
            best_R = R;
        }
    }
    if (best_R == 0) return false;
    a.R = best_R;
    a.tpi = ceil_div(c.Ho, a.R);
    a.Rin = (a.R - 1) * c.sh + c.Hf;
    a.OS = a.Rin * c.Wi;
    a.ppo = a.OS / 2;
    a.tasks = oct * a.ppo;
    a.lds_bytes = (uint32_t)(per_pixel * a.OS * 16);
    const int64_t tiles = (int64_t)c.N * a.tpi * a.co_tiles;
    if (tiles > 0x7fffffff) return false;
    const int64_t xb = (int64_t)c.N * c.Ci * c.Hi * c.Wi * 2;
    const int64_t yb = (int64_t)c.N * c.Co * c.Ho * c.Wo * 4;
    const int64_t wb = (int64_t)oct * a.HWp * a.Copad * 16;
    if (xb >= (int64_t)kMissR || yb >= (int64_t)kMissR || wb >= (int64_t)kMissR) return false;
    a.xbytes = (uint32_t)xb;
    a.ybytes = (uint32_t)yb;
    a.wbytes = (uint32_t)wb;
    a.divCoT = FastDiv((uint32_t)a.co_tiles);
    a.divTpi = FastDiv((uint32_t)a.tpi);
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divWf = FastDiv((uint32_t)c.Wf);
    a.divHW = FastDiv((uint32_t)a.HW);
    a.divPpo = FastDiv((uint32_t)a.ppo);
    a.divOCTP = FastDiv((uint32_t)a.OCTP);
    a.swz = knob(KNOB_TILE_ORDER) != 1;
    return true;
}

int nb_of(const ResArgs& a)
{
    const int need = ceil_div(a.R * a.c.Wo, 16);
    for (int v : kResNBs)
        if (v >= need) return v;
    return 0;
}

template <int NB, bool NHWC>
int launch_t(const uint16_t* x, const uint4* wpk, float* y, const ResArgs& a, hipStream_t stream)
{
    constexpr int NCB = 4;   // 8 waves, two per SIMD: 1.06x faster on cv5 than NCB = 8
    ensure_lds_limit((const void*)conv_f16_res_kernel<NB, NCB, NHWC>, kResLds);
    hipLaunchKernelGGL((conv_f16_res_kernel<NB, NCB, NHWC>),
                       dim3((unsigned)((int64_t)a.c.N * a.tpi * a.co_tiles)),
                       dim3(128 * kResCo / (16 * NCB)), a.lds_bytes, stream, x, wpk, y, a);
    return launch_status();
}

template <bool NHWC>
int launch_nb(const uint16_t* x, const uint4* wpk, float* y, const ResArgs& a, hipStream_t stream)
{
    switch (nb_of(a)) {
    case 8: return launch_t<8, NHWC>(x, wpk, y, a, stream);
    case 10: return launch_t<10, NHWC>(x, wpk, y, a, stream);
    case 13: return launch_t<13, NHWC>(x, wpk, y, a, stream);
    default: return -1;
    }
}

}  // namespace

bool f16_res_applies(const ConvShape& c, size_t copad_mult, const void* x, const void* y,
                     bool nhwc)
{
    ResArgs a;
    return (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0 && plan(c, a, copad_mult, nhwc);
}

int launch_conv_f16_res(const uint16_t* x, const void* wpk, float* y, const ConvShape& c,
                        size_t copad_mult, bool nhwc, hipStream_t stream)
{
    ResArgs a;
    if (!wpk || (uintptr_t)wpk % 16 != 0 || (uintptr_t)x % 16 != 0 || (uintptr_t)y % 16 != 0)
        return -1;
    if (!plan(c, a, copad_mult, nhwc)) return -1;
    const uint4* w4 = static_cast<const uint4*>(wpk);
    return nhwc ? launch_nb<true>(x, w4, y, a, stream) : launch_nb<false>(x, w4, y, a, stream);
}

}  // namespace im2win
