// fp16 im2win convolution on the CDNA4 matrix cores with each staged input
// row reused across the output rows that share it, and the filter held in
// registers.
//
// The half-precision path of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract:
// half-precision multiply-accumulate on matrix hardware; Fig. 1: each output
// is the dot product of a filter with one window), laid out for the im2win
// property of "Im2win: Memory Efficient Convolution On SIMD Architectures"
// (Abstract): the part of a window that lies in one input row is one
// contiguous run of that row, and the rows of consecutive output rows'
// windows overlap when the row stride is below the filter height.
//
//  * GEMM view as in the row-staged kernel: rows = output channels (A =
//    filters), K slices of 8 = (input channel c, filter row kh) with the 8
//    filter columns kw in one slice (kw >= Wf zero), so a lane's B operand of
//    v_mfma_f32_32x32x16_f16 is 8 consecutive input columns wo*sw .. +7 of
//    one input row: one 16-byte LDS read. Lanes 0-31 take channel c, lanes
//    32-63 channel c+1 of the same filter row.
//  * Output pixels are grouped in row groups of J = 4 consecutive output rows
//    of one image; the columns of all row groups of the batch are numbered
//    in a row, p = (n*G + g)*Wo + wo (G row groups per image). A lane owns
//    one column p and computes its J pixels (n, g*J + j, wo), j < J. The 4
//    accumulator blocks of a wave are those J rows of its 32 columns, so a B
//    read of relative input row R (input row g*J*SH + R) feeds the blocks j
//    with 0 <= R - j*SH < HF, each with the filter row kh = R - j*SH.
//  * Per channel pair a wave reads each of the (J-1)*SH + HF input rows it
//    needs once and holds them in registers, then takes the HF filter rows
//    in turn: filter row kh (two 32-channel fragments) multiplies input rows
//    kh + j*SH, 2*J independent MFMAs. A B read feeds up to 2*J MFMAs and an
//    A read J (cv4: 27 KB of LDS reads per 56 MFMAs, against 42 KB for the
//    row-staged kernel's 2 x 4 tiles).
//  * A workgroup of NWV waves owns 32*NWV consecutive columns (J*32*NWV
//    pixels) and 64 output channels. A stage is Cg input channels: their
//    filter slices (prepacked as [c][kh][co][8], or gathered from w) and the
//    input rows of every row group the tile touches are copied into LDS by
//    buffer_load_dwordx4 ... lds, three stage buffers rotating, loads two
//    stages ahead, one barrier per stage, as in the row-staged kernel.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "knobs.hpp"

namespace im2win {

namespace {

constexpr int kLds = 160 * 1024;
constexpr int kCoT = 64;                  // output channels per tile
constexpr int kJ = 4;                     // output rows per row group
constexpr int kBufs = 3;                  // stage buffers: loads two stages ahead
constexpr int kSlack = 2048;              // LDS past the last buffer (reads past a stage)
constexpr uint32_t kMiss = 0xFFFFFFF0u;   // vector offset past every accepted buffer

struct ReuseArgs {
    ConvShape c;
    int G;                          // row groups per image, ceil(Ho / J)
    int P, co_tiles;                // columns per tile; channel tiles
    int64_t px_tiles, cols;         // tiles; columns N*G*Wo
    int gmax, kmax, dup, RIN;       // row groups a tile touches, image breaks, halo rows per
                                    // break, LDS rows per channel
    int RP;                         // halves per LDS row (multiple of 8)
    int Cg, S, NX, NS, Copad;       // channels per stage, slices per stage (Cg*Hf), row kilobytes
                                    // per stage, stages (Ci/Cg), prepacked filter channels
    uint32_t stage_bytes;           // (S + NX) KB: filter slices, then rows
    uint32_t dummy;                 // LDS byte offset of the landing kilobyte of unused loads
    uint32_t lds_bytes;
    uint32_t xbytes, ybytes, wbytes, worig;   // x, y, prepacked filter, filter in w's layout
    uint32_t mask[4];               // halves kw >= Wf cleared (B dwords, gathered filter entries)
    bool swz;                       // XCD-grouped tile order
    bool sync;                      // stages copied through registers, one buffer
    FastDiv divWo, divG;
};

template <int NWV, int DMAX, int HF, int SH, bool WPK>
__global__ __launch_bounds__(64 * NWV) void conv_f16_reuse_kernel(const uint16_t* __restrict__ x,
                                                                  const uint4* __restrict__ wp,
                                                                  const uint16_t* __restrict__ w,
                                                                  float* __restrict__ y,
                                                                  ReuseArgs a)
{
    constexpr int NT = 64 * NWV;
    constexpr int RC = (kJ - 1) * SH + HF;   // input rows of a row group
    extern __shared__ __align__(16) unsigned char smem[];
    const uint32_t lbase =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co;
    const int sw = a.c.sw;
    const int Ho = a.c.Ho, Wo = a.c.Wo;
    const int G = a.G;

    // XCD-grouped tile order unless the tile_order knob asks for launch order.
    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x, a.swz);
    const int co_t = (int)(bid % a.co_tiles);
    const int64_t pt = bid / a.co_tiles;
    const int co0 = co_t * kCoT;
    const int64_t p0 = pt * a.P;
    const int64_t pend = p0 + a.P < a.cols ? p0 + a.P : a.cols;
    // First and last row group of the tile (numbered over the batch, n*G + g)
    // and the tile's first image.
    const int cg0 = (int)a.divWo.div((uint32_t)p0);
    const int cgl = (int)a.divWo.div((uint32_t)(pend - 1));
    const int n0 = (int)a.divG.div((uint32_t)cg0);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int wave = uniform(tid >> 6);

    // This lane's column: row group cg (image n, group g) and output column
    // wo; its row group's first input row sits at LDS row
    // (cg - cg0)*J*SH + (n - n0)*dup.
    int64_t pme = p0 + wave * 32 + l32;
    const bool pok = pme < pend;
    if (!pok) pme = pend - 1;
    const int cgme = (int)a.divWo.div((uint32_t)pme);
    const int wome = (int)(pme - (int64_t)cgme * Wo);
    const int nme = (int)a.divG.div((uint32_t)cgme);
    const int gme = cgme - nme * G;
    const int pb = (((cgme - cg0) * kJ * SH + (nme - n0) * a.dup) * a.RP + wome * sw) * 2;

    // LDS row i -> (image n, input row h); false if no input row maps there
    // (past the tile's row groups, or past the image's last row).
    auto x_src = [&](int i, int& n, int& h) -> bool {
        for (int k = 0; k <= a.kmax; ++k) {
            const int nk = n0 + k;
            const int first = max(cg0, nk * G), last = min(cgl, nk * G + G - 1);
            if (first > last) break;
            const int S0 = (first - cg0) * kJ * SH + k * a.dup;
            const int span = (last - first) * kJ * SH + RC;
            if (i >= S0 && i < S0 + span) {
                n = nk;
                h = (first - nk * G) * kJ * SH + (i - S0);
                return h < Hi;
            }
        }
        return false;
    };

    // Input columns the tile reads in row h of image n: the union, over the
    // row groups of the tile that use the row, of [wa*sw, (wb-1)*sw + 8) for
    // the tile's output columns [wa, wb) of that group. Chunks outside are
    // not fetched (their LDS entries read as zeros and no lane reads them).
    auto x_cols = [&](int n, int h, int& c0, int& c1) {
        c0 = 1 << 30;
        c1 = 0;
        const int step = kJ * SH;
        const int glo = max(0, (h - RC + step) / step), ghi = min(G - 1, h / step);
        for (int g = glo; g <= ghi; ++g) {
            const int64_t cg = (int64_t)n * G + g;
            const int64_t qa = max(p0, cg * Wo), qb = min(pend, (cg + 1) * Wo);
            if (qa >= qb) continue;
            c0 = min(c0, (int)(qa - cg * Wo) * sw);
            c1 = max(c1, (int)(qb - 1 - cg * Wo) * sw + 8);
        }
    };

    // Load slots of a stage: slot m < S is filter slice m (one kilobyte: the
    // tile's 64 channels), slot S + j is kilobyte j of the stage's rows, later
    // slots land in the dummy kilobyte. Wave v issues slots v + NWV*i; the
    // per-lane offsets do not depend on the stage (its channels enter through
    // the buffer base), so they are worked out once.
    uint32_t voff[DMAX];
    const int rpc = a.RP >> 3;   // 16-byte chunks per LDS row
#pragma unroll
    for (int i = 0; i < DMAX; ++i) {
        const int m = wave + NWV * i;
        uint32_t v = kMiss;
        if (m < a.S) {
            if (WPK) v = (uint32_t)(((m * a.Copad + co0) + lane) * 16);
        } else if (m < a.S + a.NX) {
            const int e = (m - a.S) * 64 + lane;
            const int row = e / rpc, cc = e - row * rpc;
            const int cl = row / a.RIN, r = row - cl * a.RIN;
            int n, h, c0, c1;
            if (cl < a.Cg && 8 * cc < Wi && x_src(r, n, h)) {
                x_cols(n, h, c0, c1);
                if (8 * cc + 8 > c0 && 8 * cc < c1)
                    v = (uint32_t)(((((int64_t)n * Ci + cl) * Hi + h) * Wi + 8 * cc) * 2);
            }
        }
        voff[i] = v;
    }
    auto issue = [&](int s, int sb) {
        const uint32_t fo = (uint32_t)s * a.S * a.Copad * 16;
        const int64_t xo = (int64_t)s * a.Cg * Hi * Wi;
        const __amdgpu_buffer_rsrc_t ra =
            raw_rsrc(wp + (int64_t)s * a.S * a.Copad, WPK ? a.wbytes - fo : 0u);
        const __amdgpu_buffer_rsrc_t rx = raw_rsrc(x + xo, a.xbytes - (uint32_t)(xo * 2));
        const uint32_t base = lbase + (uint32_t)sb * a.stage_bytes;
#pragma unroll
        for (int i = 0; i < DMAX; ++i) {
            const int m = wave + NWV * i;
            const bool real = m < a.S + a.NX && (WPK || m >= a.S);
            const uint32_t dst = real ? base + (uint32_t)m * 1024 : lbase + a.dummy;
            lds_dma16(m < a.S ? ra : rx, dst, voff[i]);
        }
    };
    auto issue_none = [&]() {
        const __amdgpu_buffer_rsrc_t rx = raw_rsrc(x, a.xbytes);
#pragma unroll
        for (int i = 0; i < DMAX; ++i) lds_dma16(rx, lbase + a.dummy, kMiss);
    };
    // Without direct loads (sync): the same slots copied through registers
    // into buffer sb, four slots at a time, each wave waiting for its loads.
    auto copy_stage = [&](int s, int sb) {
        const uint32_t fo = (uint32_t)s * a.S * a.Copad * 16;
        const int64_t xo = (int64_t)s * a.Cg * Hi * Wi;
        const __amdgpu_buffer_rsrc_t ra =
            raw_rsrc(wp + (int64_t)s * a.S * a.Copad, WPK ? a.wbytes - fo : 0u);
        const __amdgpu_buffer_rsrc_t rx = raw_rsrc(x + xo, a.xbytes - (uint32_t)(xo * 2));
        unsigned char* base = smem + (size_t)sb * a.stage_bytes;
#pragma unroll
        for (int i0 = 0; i0 < DMAX; i0 += 4) {
            uint4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int m = wave + NWV * (i0 + k);
                if (i0 + k < DMAX) {
                    const auto r = __builtin_amdgcn_raw_buffer_load_b128(m < a.S ? ra : rx,
                                                                         (int)voff[i0 + k], 0, 0);
                    v[k] = make_uint4(r[0], r[1], r[2], r[3]);
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int m = wave + NWV * (i0 + k);
                if (i0 + k < DMAX && m < a.S + a.NX && (WPK || m >= a.S))
                    *reinterpret_cast<uint4*>(base + (size_t)m * 1024 + 16 * lane) = v[k];
            }
        }
    };

    floatx16_t acc[2][kJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const uint32_t m0 = a.mask[0], m1 = a.mask[1], m2 = a.mask[2], m3 = a.mask[3];
    const int rp2 = a.RP * 2;
    const int cstride = a.RIN * rp2;   // bytes between a stage's channels in LDS

    // The MFMAs of channel pair cp of the stage in buffer (A: filter slices,
    // X: rows). Filter fragment (block i, row kh): lanes 0-31 the entry of
    // slice (2cp, kh), lanes 32-63 of slice (2cp+1, kh), channel i*32 + l32.
    auto pair_mmas = [&](const unsigned char* A, const unsigned char* X, int cp) {
        // Filter-row-major order: step kh multiplies the two fragments of
        // filter row kh with the input rows R = kh + j*SH of the J output
        // rows, 2*J MFMAs into 2*J different accumulators, so no MFMA waits
        // for the one before it. The RC input-row fragments are read once
        // (in the order the steps first need them) and held, masked, in
        // registers; the filter fragments of step kh+1 are read during step
        // kh. Scheduling barriers keep the compiler from moving reads next
        // to their first use.
        half8_t bq[RC];
        half8_t af[2][2];
        const unsigned char* Ab = A + (size_t)((2 * cp + hl) * HF * kCoT + l32) * 16;
        const unsigned char* B = X + (2 * cp + hl) * cstride + pb;
        auto read_a = [&](int kh) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                __builtin_memcpy(&af[kh & 1][i], Ab + (size_t)(kh * kCoT + i * 32) * 16, 16);
        };
        // B addresses are 4-byte aligned (even column stride, row pitch a
        // multiple of 8 halves); stated so, the reads become aligned
        // dword-pair reads instead of the slower unaligned 16-byte form.
        auto read_b = [&](int R) {
            __builtin_memcpy(&bq[R], __builtin_assume_aligned(B + R * rp2, 4), 16);
        };
        // Padded taps (kw >= Wf) are cleared so an infinity next to a window
        // never meets a zero filter tap.
        auto mask_b = [&](int R) {
            uint4 u;
            __builtin_memcpy(&u, &bq[R], 16);
            u.x &= m0;
            u.y &= m1;
            u.z &= m2;
            u.w &= m3;
            __builtin_memcpy(&bq[R], &u, 16);
        };
        // First needed at step kh: the rows kh + j*SH not needed before.
        auto first_step = [](int R) {
            int f = HF;
#pragma unroll
            for (int j = 0; j < kJ; ++j)
                if (R - j * SH >= 0 && R - j * SH < HF && R - j * SH < f) f = R - j * SH;
            return f;
        };
        read_a(0);
#pragma unroll
        for (int R = 0; R < RC; ++R)
            if (first_step(R) == 0) read_b(R);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kh = 0; kh < HF; ++kh) {
            if (kh + 1 < HF) {
                read_a(kh + 1);
#pragma unroll
                for (int R = 0; R < RC; ++R)
                    if (first_step(R) == kh + 1) read_b(R);
            }
#pragma unroll
            for (int R = 0; R < RC; ++R)
                if (first_step(R) == kh) mask_b(R);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kJ; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[kh & 1][i],
                                                                       bq[kh + j * SH], acc[i][j],
                                                                       0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Without a prepacked filter: entry e = (slice m, channel co0 + j), m =
    // e / 64, j = e % 64, of stage sg holds the taps of
    // w[co0 + j][sg*Cg + m/HF][m%HF][*] (zeros past Wf and Co), one run of
    // Wf halves. Each thread builds kGE entries whole: a 16-byte load from
    // the dword boundary at or below the run (and the next dword when Wf =
    // 8) holds it, shifted down 2 bytes when the run starts between dwords;
    // the halves kw >= Wf are cleared. A wave's 64 lanes take 16 consecutive
    // channels x 4 consecutive slices (entry_of), so its loads touch few
    // cache lines and each 8 lanes write 128 consecutive LDS bytes. w is
    // read through a buffer that starts at the dword boundary at or below it;
    // an entry whose loads would reach past w's end (only w's last run)
    // takes its taps one by one. The loads of stage s+2 go out with stage
    // s's direct loads and are written after its MFMAs.
    // Entries per thread and stage: S = Cg*HF <= 4*HF slices of 64 entries
    // over NT threads.
    constexpr int kGE = (4 * HF + NWV - 1) / NWV;
    uint4 gu[kGE];
    uint32_t gt[kGE], gs[kGE];
    const uint32_t wal = (uint32_t)((uintptr_t)w & 3);
    const uint32_t wrng = a.worig + wal;
    // Byte offset in w of entry e's run in stage sg; kMiss past the stage's
    // entries and channels.
    // Entry k of this thread: lane l of wave v takes channel 16(v % 4) +
    // l % 16 of slice 4(v / 4) + l / 16 + 8k (8 waves: slices 8k .. 8k+7).
    static_assert(NWV % 4 == 0, "entry_of spreads 64 channels over groups of 4 waves");
    auto entry_of = [&](int k) -> int {
        const int lane = tid & 63, v = tid >> 6;
        const int j = (lane & 15) + 16 * (v & 3);
        const int m = (lane >> 4) + 4 * (v >> 2) + 4 * (NWV / 4) * k;
        return m * 64 + j;
    };
    auto entry_src = [&](int sg, int e) -> uint32_t {
        const int m = e >> 6, co = co0 + (e & 63);
        const int c = sg * a.Cg + m / HF, kh = m - (m / HF) * HF;
        return e < a.S * 64 && co < Co ? (uint32_t)((((co * Ci + c) * HF + kh) * a.c.Wf) * 2)
                                       : kMiss;
    };
    auto gather_load = [&](int sg) {
        const __amdgpu_buffer_rsrc_t ra =
            raw_rsrc(reinterpret_cast<const unsigned char*>(w) - wal, wrng);
#pragma unroll
        for (int k = 0; k < kGE; ++k) {
            const uint32_t src = entry_src(sg, entry_of(k));
            const uint32_t sa = (src + wal) & ~3u;
            const bool tail = src != kMiss && sa + 20 > wrng;
            const bool hit = src != kMiss && !tail;
            const auto u = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(hit ? sa : kMiss), 0, 0);
            gu[k] = make_uint4(u[0], u[1], u[2], u[3]);
            gt[k] = a.c.Wf == 8 ? __builtin_amdgcn_raw_buffer_load_b32(
                                      ra, (int)(hit ? sa + 16 : kMiss), 0, 0)
                                : 0u;
            gs[k] = tail ? 1u : ((src + wal) & 2u) * 8u;
        }
    };
    auto gather_store = [&](int sg, int sb) {
        uint4* F = reinterpret_cast<uint4*>(smem + (size_t)sb * a.stage_bytes);
        const __amdgpu_buffer_rsrc_t rw = raw_rsrc(w, a.worig);
#pragma unroll
        for (int k = 0; k < kGE; ++k) {
            const int e = entry_of(k);
            if (e >= a.S * 64) continue;
            uint4 v;
            if (gs[k] == 1u) {   // w's last run: tap by tap
                const uint32_t src = entry_src(sg, e);
                uint32_t hv[8];
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    hv[q] = __builtin_amdgcn_raw_buffer_load_b16(
                        rw, (int)(q < a.c.Wf ? src + 2 * q : kMiss), 0, 0);
                v = make_uint4(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                               hv[6] | (hv[7] << 16));
            } else {
                const uint4 u = gu[k];
                v = make_uint4(__builtin_amdgcn_alignbit(u.y, u.x, gs[k]),
                               __builtin_amdgcn_alignbit(u.z, u.y, gs[k]),
                               __builtin_amdgcn_alignbit(u.w, u.z, gs[k]),
                               __builtin_amdgcn_alignbit(gt[k], u.w, gs[k]));
            }
            v.x &= m0;
            v.y &= m1;
            v.z &= m2;
            v.w &= m3;
            F[e] = v;
        }
    };

    // sync: one buffer, each stage copied through registers after every
    // wave is done with the one before, and computed once it has landed (no
    // copy in flight during the MFMAs).
    const bool sync = a.sync;
    if (!sync) {
        issue(0, 0);
        if (a.NS > 1) issue(1, 1); else issue_none();
        if (!WPK) {
            gather_load(0);
            gather_store(0, 0);
            if (a.NS > 1) {
                gather_load(1);
                gather_store(1, 1);
            }
        }
    }
    const int npairs = a.Cg >> 1;
    for (int s = 0; s < a.NS; ++s) {
        if (sync) {
            __syncthreads();   // every wave is done with the previous stage
            copy_stage(s, 0);
            if (!WPK) {
                gather_load(s);
                gather_store(s, 0);
            }
            __syncthreads();
        } else {
            // This wave's loads of stage s have landed (those of stage s+1
            // may still be in flight).
            wait_vm<DMAX>();
            __syncthreads();      // every wave's; and stage s-1's buffer is free
            if (s + 2 < a.NS) issue(s + 2, (s + 2) % kBufs); else issue_none();
            if (!WPK && s + 2 < a.NS) gather_load(s + 2);
        }
        const unsigned char* A = smem + (size_t)(sync ? 0 : s % kBufs) * a.stage_bytes;
        const unsigned char* X = A + (size_t)a.S * 1024;
        for (int cp = 0; cp < npairs; ++cp) pair_mmas(A, X, cp);
        // Stage s+2's buffer was freed by the barrier above.
        if (!sync && !WPK && s + 2 < a.NS) gather_store(s + 2, (s + 2) % kBufs);
    }
    wait_vm<0>();   // the last (unused) loads have landed before the workgroup ends

    // Output: lane holds, for each of its J pixels (n, g*J + j, wo), channels
    // 8*(r/4) + 4*hl + r%4 of each 32-channel block; every store writes 32
    // consecutive pixels of one output row into each of two channel planes.
    if (!pok) return;
    const int64_t plane = (int64_t)Ho * Wo;
    const __amdgpu_buffer_rsrc_t yb = raw_rsrc(y, a.ybytes);
    const bool all_co = co0 + kCoT <= Co;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
        const int ho = gme * kJ + j;
        if (ho >= Ho) break;
        const uint32_t vo =
            (uint32_t)((((int64_t)nme * Co + 4 * hl) * plane + (int64_t)ho * Wo + wome) * 4);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int cu = co0 + i * 32 + 8 * (r >> 2) + (r & 3);   // channel - 4*hl
                if (all_co || cu + 4 * hl < Co)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), yb,
                                                          (int)vo, (int)(cu * plane * 4), 0);
            }
    }
}

// Load instructions per wave and stage the kernel is built for.
constexpr int kDmax[] = {4, 6, 8, 12, 16};
// (filter height, row stride) pairs it is built for.
constexpr int kShapes[][2] = {{7, 2}, {5, 2}, {3, 2}, {3, 1}, {5, 1}, {7, 1}};

bool shape_built(int hf, int sh)
{
    for (const auto& p : kShapes)
        if (p[0] == hf && p[1] == sh) return true;
    return false;
}

// Plans a launch; false if the shape is outside the kernel's envelope: even
// column stride, Wf <= 8, Wi a multiple of 8 (16-byte row chunks), even Ci,
// a (filter height, row stride) pair the kernel is built for, a stage of at
// least two channels in LDS, tensors addressable with 32-bit buffer offsets.
// Knobs: KNOB_F16_REUSE < 0 turns the kernel off; KNOB_TILE_ORDER = 1 keeps
// tiles in launch order.
bool plan(const ConvShape& c, ReuseArgs& a, int& nwv, int& dmax)
{
    if (knob(KNOB_F16_REUSE) < 0 || knob(KNOB_F16_ROWS) < 0) return false;
    if (c.Wf > 8 || c.sw % 2 != 0 || c.Wi % 8 != 0 || c.Ci % 2 != 0) return false;
    if (!shape_built(c.Hf, c.sh)) return false;
    a.c = c;
    a.G = ceil_div(c.Ho, kJ);
    const int RC = (kJ - 1) * c.sh + c.Hf;
    a.dup = std::max(0, RC - kJ * c.sh);
    a.cols = (int64_t)c.N * a.G * c.Wo;
    if (a.cols >= 0x7fffffff || (int64_t)c.N * a.G >= 0x7fffffff) return false;
    a.RP = ((std::max(c.Wi, (c.Wo - 1) * c.sw + 8) + 7) / 8) * 8;
    a.Copad = ceil_div(c.Co, kCoT) * kCoT;
    nwv = 8;
    a.P = 32 * nwv;
    // Row groups a tile touches (never more than the batch has) and image
    // breaks inside a tile (never more than N - 1).
    a.gmax = (int)std::min<int64_t>((a.P - 1) / c.Wo + 2, (int64_t)c.N * a.G);
    const int64_t gcols = (int64_t)a.G * c.Wo;   // columns per image
    a.kmax = a.gmax <= 1 ? 0 : (int)std::min<int64_t>(c.N - 1, (a.P - 1) / gcols + 1);
    a.RIN = (a.gmax - 1) * kJ * c.sh + RC + a.kmax * a.dup;
    bool found = false;
    for (int cg : {4, 2}) {
        if (c.Ci % cg != 0) continue;
        const int S = cg * c.Hf;
        const int NX = (int)ceil_div(cg * a.RIN * a.RP * 2, 1024);
        const int need = ceil_div(S + NX, nwv);
        int dm = 0;
        for (int d : kDmax)
            if (d >= need) {
                dm = d;
                break;
            }
        if (!dm) continue;
        const int64_t stage = (int64_t)(S + NX) * 1024;
        const int64_t lds = kBufs * stage + 1024 + kSlack;
        if (lds > kLds || S > (4 * c.Hf + nwv - 1) / nwv * nwv) continue;   // gather entries

        a.Cg = cg;
        a.S = S;
        a.NX = NX;
        a.stage_bytes = (uint32_t)stage;
        a.dummy = (uint32_t)(kBufs * stage);
        a.lds_bytes = (uint32_t)lds;
        dmax = dm;
        found = true;
        break;
    }
    if (!found) return false;
    a.NS = c.Ci / a.Cg;
    a.co_tiles = ceil_div(c.Co, kCoT);
    a.px_tiles = (a.cols + a.P - 1) / a.P;
    if (a.px_tiles * a.co_tiles > 0x7fffffff) return false;
    // Buffer ranges are 32-bit and the miss offset must lie past every one.
    const int64_t xb = (int64_t)c.N * c.Ci * c.Hi * c.Wi * 2;
    const int64_t yb = (int64_t)c.N * c.Co * c.Ho * c.Wo * 4;
    const int64_t wb = (int64_t)c.Ci * c.Hf * a.Copad * 16;
    const int64_t wo = (int64_t)c.Co * c.Ci * c.Hf * c.Wf * 2;
    if (xb >= 0x7fffffff || yb >= (int64_t)kMiss || wb >= 0x7fffffff || wo >= 0x7fffffff)
        return false;
    a.worig = (uint32_t)wo;
    a.xbytes = (uint32_t)xb;
    a.ybytes = (uint32_t)yb;
    a.wbytes = (uint32_t)wb;
    for (int d = 0; d < 4; ++d) {
        uint32_t m = 0;
        if (2 * d < c.Wf) m |= 0xFFFFu;
        if (2 * d + 1 < c.Wf) m |= 0xFFFF0000u;
        a.mask[d] = m;
    }
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divG = FastDiv((uint32_t)a.G);
    a.swz = knob(KNOB_TILE_ORDER) != 1;
    a.sync = knob(KNOB_SYNC_STAGING) == 1;
    return true;
}

template <int NWV, int DMAX, int HF, int SH, bool WPK>
int launch_t(const uint16_t* x, const uint4* wp, const uint16_t* w, float* y, const ReuseArgs& a,
             hipStream_t stream)
{
    ensure_lds_limit((const void*)conv_f16_reuse_kernel<NWV, DMAX, HF, SH, WPK>, kLds);
    hipLaunchKernelGGL((conv_f16_reuse_kernel<NWV, DMAX, HF, SH, WPK>),
                       dim3((unsigned)(a.px_tiles * a.co_tiles)), dim3(64 * NWV), a.lds_bytes,
                       stream, x, wp, w, y, a);
    return launch_status();
}

template <int HF, int SH, bool WPK>
int launch_d(int dmax, const uint16_t* x, const uint4* wp, const uint16_t* w, float* y,
             const ReuseArgs& a, hipStream_t stream)
{
    switch (dmax) {
    case 4: return launch_t<8, 4, HF, SH, WPK>(x, wp, w, y, a, stream);
    case 6: return launch_t<8, 6, HF, SH, WPK>(x, wp, w, y, a, stream);
    case 8: return launch_t<8, 8, HF, SH, WPK>(x, wp, w, y, a, stream);
    case 12: return launch_t<8, 12, HF, SH, WPK>(x, wp, w, y, a, stream);
    case 16: return launch_t<8, 16, HF, SH, WPK>(x, wp, w, y, a, stream);
    }
    return -1;
}

template <bool WPK>
int launch_s(int dmax, const uint16_t* x, const uint4* wp, const uint16_t* w, float* y,
             const ReuseArgs& a, hipStream_t stream)
{
    const int hf = a.c.Hf, sh = a.c.sh;
    if (hf == 7 && sh == 2) return launch_d<7, 2, WPK>(dmax, x, wp, w, y, a, stream);
    if (hf == 5 && sh == 2) return launch_d<5, 2, WPK>(dmax, x, wp, w, y, a, stream);
    if (hf == 3 && sh == 2) return launch_d<3, 2, WPK>(dmax, x, wp, w, y, a, stream);
    if (hf == 3 && sh == 1) return launch_d<3, 1, WPK>(dmax, x, wp, w, y, a, stream);
    if (hf == 5 && sh == 1) return launch_d<5, 1, WPK>(dmax, x, wp, w, y, a, stream);
    if (hf == 7 && sh == 1) return launch_d<7, 1, WPK>(dmax, x, wp, w, y, a, stream);
    return -1;
}

}  // namespace

bool f16_reuse_applies(const ConvShape& c)
{
    ReuseArgs a;
    int nwv, dmax;
    return plan(c, a, nwv, dmax);
}

int launch_conv_f16_reuse(const uint16_t* x, const void* wp, const uint16_t* w, float* y,
                          const ConvShape& c, hipStream_t stream)
{
    ReuseArgs a;
    int nwv, dmax;
    if (!plan(c, a, nwv, dmax)) return -1;
    // Rows are fetched in 16-byte chunks from 16-byte boundaries.
    if ((uintptr_t)x % 16 != 0 || (uintptr_t)wp % 16 != 0) return -1;
    const uint4* w4 = static_cast<const uint4*>(wp);
    return w4 ? launch_s<true>(dmax, x, w4, w, y, a, stream)
              : launch_s<false>(dmax, x, w4, w, y, a, stream);
}

}  // namespace im2win
