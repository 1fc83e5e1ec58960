// fp16 convolution from the materialised im2win tensor on the CDNA4 matrix
// cores.
//
// The formulation of "Im2win: Memory Efficient Convolution On SIMD
// Architectures" (Abstract) and "Enabling Memory-efficient Im2win
// Convolution with Multi-precision Support on GPU CUDA and Tensor Cores"
// (Fig. 1, middle; Abstract: half precision on matrix hardware): the window
// of output (n, ho, wo) in input channel c is the one contiguous run of Wf*Hf
// elements ws[n][c][ho][wo*sw*Hf ...] of the packed tensor, in window order
// j = kw*Hf + kh, and every output is the dot product of those runs with the
// filter taps in the same order.
//
//  * GEMM view: rows = output channels (A = filters), columns = output
//    pixels numbered over the batch, q = (n*Ho + ho)*Wo + wo (B = windows),
//    K = (input channel c, window position j) with each channel's Wf*Hf
//    positions padded to M slices of 8. Slice m of a pixel's window is the 8
//    consecutive elements wo*sw*Hf + 8m .. +7 of its row: one 16-byte LDS
//    read per lane for v_mfma_f32_32x32x16_f16 (lanes 0-31 slice 2t, 32-63
//    slice 2t+1 of the stage). Positions past Wf*Hf in a channel's last slice
//    are zero in the filter and masked to zero in B.
//  * The pixels of a tile are consecutive, so in each (image, channel) plane
//    their windows lie in one contiguous stretch of the packed tensor
//    (output rows follow each other in the plane). A stage copies that
//    stretch for Cg channels into LDS with buffer_load_dwordx4 ... lds (16
//    bytes per lane straight into LDS), a separate stretch per image when a
//    tile crosses images, and gathers the stage's filter slices from w into
//    LDS in window order, each thread building whole 16-byte entries from
//    two-byte loads after the stage before it. Two stage buffers alternate:
//    the next stage's loads go out as a stage starts, one barrier per stage.
//  * A workgroup of NWV waves owns 64 output channels and 128*NWV pixels;
//    each wave a 2 x 4 register tile of 32 x 32 accumulators (64 channels x
//    128 pixels), so every A read feeds four MFMAs and every B read two.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "knobs.hpp"

namespace im2win {

namespace {

template <int K>
struct IC {
    static constexpr int value = K;
};

constexpr int kWsLds = 160 * 1024;
constexpr int kCoT = 64;                  // output channels per tile
constexpr int kNB = 4;                    // 32-pixel blocks per wave
constexpr int kBufs = 2;                  // stage buffers: loads one stage ahead
constexpr int kSlack = 2048;              // LDS past the last buffer (reads past a stage)
constexpr uint32_t kMiss = 0xFFFFFFF0u;   // vector offset past every accepted buffer
constexpr int kMaxSeg = 4;                // images a tile may touch

struct WsArgs {
    ConvShape c;
    int P, co_tiles;
    int64_t px_tiles, total;
    int M;                          // slices per channel, ceil(Hf*Wf / 8)
    int L, step;                    // packed row length Wi*Hf; window start step sw*Hf
    int kmax;                       // image breaks inside a tile
    int XC;                         // LDS halves per channel region (multiple of 8)
    int Cg, S, NX, NS;              // channels per stage, slices per stage (Cg*M), region
                                    // kilobytes per stage, stages
    uint32_t stage_bytes;           // (S + NX) KB: filter slices, then the channels' regions
    uint32_t dummy;                 // LDS byte offset of the landing kilobyte of unused loads
    uint32_t lds_bytes;
    uint32_t wsbytes, ybytes, worig;
    uint32_t lastmask[4];           // B dwords of a channel's last slice: positions past Wf*Hf cleared
    bool swz;                       // XCD-grouped tile order
    bool sync;                      // stages copied through registers, one buffer
    FastDiv divWo, divHo, divPlane;
};




template <int NWV, int DMAX, bool ODD>
__global__ __launch_bounds__(64 * NWV) void conv_f16_ws_kernel(const uint16_t* __restrict__ ws,
                                                               const uint16_t* __restrict__ w,
                                                               float* __restrict__ y, WsArgs a)
{
    constexpr int NT = 64 * NWV;
    extern __shared__ __align__(16) unsigned char smem[];
    const uint32_t lbase =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

    const int Ci = a.c.Ci, Co = a.c.Co, Hf = a.c.Hf, Wf = a.c.Wf;
    const int Ho = a.c.Ho, Wo = a.c.Wo;
    const int HW = Hf * Wf, M = a.M, L = a.L, step = a.step;
    const int64_t plane = (int64_t)Ho * Wo;

    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x, a.swz);
    const int co_t = (int)(bid % a.co_tiles);
    const int64_t pt = bid / a.co_tiles;
    const int co0 = co_t * kCoT;
    const int64_t q0 = pt * a.P;
    const int64_t qend = q0 + a.P < a.total ? q0 + a.P : a.total;
    const int n0 = (int)a.divPlane.div((uint32_t)q0);
    const int nl = (int)a.divPlane.div((uint32_t)(qend - 1));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int wave = uniform(tid >> 6);

    // Segment k (image n0 + k) of a channel region: the packed elements
    // [sa_k, sb_k) of the (image, channel) plane, at halves [off_k,
    // off_k + sb_k - sa_k) of the region. Bounds are rounded out to 8.
    int sa[kMaxSeg], off[kMaxSeg + 1];
    off[0] = 0;
#pragma unroll
    for (int k = 0; k < kMaxSeg; ++k) {
        const int n = n0 + k;
        int len = 0;
        sa[k] = 0;
        if (n <= nl) {
            const int64_t qa = max(q0, (int64_t)n * plane), qb = min(qend, (int64_t)(n + 1) * plane);
            const int pa = (int)(qa - (int64_t)n * plane), pb_ = (int)(qb - 1 - (int64_t)n * plane);
            const int hoa = (int)a.divWo.div((uint32_t)pa), wa = pa - hoa * Wo;
            const int hob = (int)a.divWo.div((uint32_t)pb_), wb = pb_ - hob * Wo;
            const int s0 = (hoa * L + wa * step) & ~7;
            const int s1 = (hob * L + wb * step + HW + 7) & ~7;
            sa[k] = s0;
            len = s1 - s0;
        }
        off[k + 1] = off[k] + len;
    }

    // Byte offset of each pixel's window (channel 0) within a stage's regions.
    int pbo[kNB];
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
        int64_t q = q0 + (wave * kNB + b) * 32 + l32;
        if (q >= qend) q = qend - 1;
        const int n = (int)a.divPlane.div((uint32_t)q);
        const int p = (int)(q - (int64_t)n * plane);
        const int ho = (int)a.divWo.div((uint32_t)p), wo = p - ho * Wo;
        const int k = n - n0;
        int o = 0, s = 0;
#pragma unroll
        for (int kk = 0; kk < kMaxSeg; ++kk)
            if (kk == k) {
                o = off[kk];
                s = sa[kk];
            }
        pbo[b] = (o + ho * L + wo * step - s) * 2;
    }
    // Odd sw*Hf: a window may start on an odd element (two bytes past a
    // dword). Its 16 bytes are then read as the five dwords around them and
    // shifted down by psh bits (0 or 16) per dword pair.
    int psh[kNB];
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
        psh[b] = ODD ? (pbo[b] & 2) * 8 : 0;
        if (ODD) pbo[b] &= ~3;
    }

    // Load slots of a stage: slot j < NX is kilobyte j of the stage's
    // channel regions (channel cl at halves cl*XC; LDS kilobyte S + j of the
    // stage buffer); later slots land in the dummy kilobyte. Wave v issues
    // slots v + NWV*i; the per-lane offsets (within the stage's first
    // channel's planes) do not depend on the stage.
    uint32_t voff[DMAX];
    const int cpc = a.XC >> 3;   // 16-byte chunks per channel region
#pragma unroll
    for (int i = 0; i < DMAX; ++i) {
        const int m = wave + NWV * i;
        uint32_t v = kMiss;
        if (m < a.NX) {
            const int e = m * 64 + lane;
            const int cl = e / cpc, h = (e - cl * cpc) * 8;   // halves into the region
            if (cl < a.Cg) {
#pragma unroll
                for (int k = 0; k < kMaxSeg; ++k)
                    if (h >= off[k] && h < off[k + 1])
                        v = (uint32_t)(((((int64_t)(n0 + k) * Ci + cl) * Ho) * L + sa[k] +
                                        (h - off[k])) * 2);
            }
        }
        voff[i] = v;
    }
    auto issue = [&](int s, int sb) {
        const int64_t xo = (int64_t)s * a.Cg * Ho * L;
        const __amdgpu_buffer_rsrc_t rx = raw_rsrc(ws + xo, a.wsbytes - (uint32_t)(xo * 2));
        const uint32_t base = lbase + (uint32_t)sb * a.stage_bytes;
#pragma unroll
        for (int i = 0; i < DMAX; ++i) {
            const int m = wave + NWV * i;
            lds_dma16(rx, m < a.NX ? base + (uint32_t)(a.S + m) * 1024 : lbase + a.dummy, voff[i]);
        }
    };
    auto issue_none = [&]() {
        const __amdgpu_buffer_rsrc_t rx = raw_rsrc(ws, a.wsbytes);
#pragma unroll
        for (int i = 0; i < DMAX; ++i) lds_dma16(rx, lbase + a.dummy, kMiss);
    };
    // Without direct loads (sync): the same row kilobytes copied through
    // registers into buffer sb, four at a time.
    auto copy_stage = [&](int s, int sb) {
        const int64_t xo = (int64_t)s * a.Cg * Ho * L;
        const __amdgpu_buffer_rsrc_t rx = raw_rsrc(ws + xo, a.wsbytes - (uint32_t)(xo * 2));
        unsigned char* base = smem + (size_t)sb * a.stage_bytes + (size_t)a.S * 1024 + 16 * lane;
#pragma unroll
        for (int i0 = 0; i0 < DMAX; i0 += 4) {
            uint4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (i0 + k < DMAX) {
                    const auto r = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)voff[i0 + k], 0, 0);
                    v[k] = make_uint4(r[0], r[1], r[2], r[3]);
                }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int m = wave + NWV * (i0 + k);
                if (i0 + k < DMAX && m < a.NX)
                    *reinterpret_cast<uint4*>(base + (size_t)m * 1024) = v[k];
            }
        }
    };

    // Filter slices of stage sg in window order: entry (slice m, channel
    // co0 + e) holds w[co0 + e][sg*Cg + m/M][kh][kw] at position p of the
    // slice for window position jj = 8*(m % M) + p = kw*Hf + kh (zeros past
    // Wf*Hf and past Co). gather_load issues the 2-byte loads of a thread's
    // first entry (for the next stage, before this stage's MFMAs, so their
    // latency is covered; the registers for more are not there);
    // gather_store loads the rest and writes them all.
    // The early loads need registers the 4-wave form and the forms with
    // more than 10 direct loads per wave do not have.
    constexpr bool kPre = NWV == 8 && DMAX <= 10;
    uint32_t hv[2][8];
    auto entry_loads = [&](int sg, int e, auto K) __attribute__((always_inline)) {
        constexpr int k = decltype(K)::value;
        const __amdgpu_buffer_rsrc_t rw = raw_rsrc(w, a.worig);
        const int m = e >> 6, co = co0 + (e & 63);
        const int cl = m / M, ms = m - cl * M;
        const int c = sg * a.Cg + cl;
        const bool ok = e < a.S * 64 && co < Co;
        const uint32_t base = (uint32_t)(((int64_t)co * Ci + c) * HW * 2);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int jj = 8 * ms + p;
            const int kw = jj / Hf, kh = jj - kw * Hf;
            hv[k][p] = __builtin_amdgcn_raw_buffer_load_b16(
                rw, (int)(ok && jj < HW ? base + (uint32_t)(kh * Wf + kw) * 2 : kMiss), 0, 0);
        }
    };
    auto gather_load = [&](int sg) __attribute__((always_inline)) {
        entry_loads(sg, tid, IC<0>{});
    };
    auto gather_store = [&](int sg, int sb) __attribute__((always_inline)) {
        uint4* F = reinterpret_cast<uint4*>(smem + (size_t)sb * a.stage_bytes);
        const int ne = a.S * 64;
        for (int e0 = 0; e0 < ne; e0 += 2 * NT) {
            if (e0 > 0) entry_loads(sg, e0 + tid, IC<0>{});
            entry_loads(sg, e0 + NT + tid, IC<1>{});
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int e = e0 + k * NT + tid;
                if (e < ne)
                    F[e] = make_uint4(hv[k][0] | (hv[k][1] << 16), hv[k][2] | (hv[k][3] << 16),
                                      hv[k][4] | (hv[k][5] << 16), hv[k][6] | (hv[k][7] << 16));
            }
        }
    };
    auto gather = [&](int sg, int sb) __attribute__((always_inline)) {
        gather_load(sg);
        gather_store(sg, sb);
    };

    floatx16_t acc[2][kNB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int b = 0; b < kNB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][b][r] = 0.f;

    struct Frags {
        half8_t a[2], b[kNB];
        bool last;   // the lane's slice is its channel's last
    };
    const uint32_t lm0 = a.lastmask[0], lm1 = a.lastmask[1], lm2 = a.lastmask[2],
                   lm3 = a.lastmask[3];
    const int abase = hl * kCoT + l32;   // A entry of slice hl, channel l32
    const int xc2 = a.XC * 2;
    // This lane's slice 2t + hl = (channel cl, slice ms) sits at byte
    // cl*XC*2 + 16*ms from a pixel's window start; it advances by two slices
    // per pair, carrying ms into cl.
    // The loop below reads one pair past a stage (never used); such a read,
    // a channel region past the stage's last, is sent back to offset 0 so
    // that every LDS read stays inside the stage's regions.
    const int oend = a.Cg * xc2;
    int sms = 0, soff = 0;
    auto fetch = [&](Frags& f, const unsigned char* A, const unsigned char* X, int t) {
        const int o = soff < oend ? soff : 0;
        f.last = sms == M - 1;
        sms += 2;
        soff += 32;
        if (sms >= M) { sms -= M; soff += xc2 - 16 * M; }
        if (sms >= M) { sms -= M; soff += xc2 - 16 * M; }
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_memcpy(&f.a[i], A + (size_t)(abase + 2 * t * kCoT + i * 32) * 16, 16);
        // B addresses are 4-byte aligned (pbo is, and regions start on
        // 16-byte boundaries); stated so, the reads become aligned dword
        // reads instead of the much slower unaligned 16-byte form.
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            if (ODD) {
                uint32_t d[5], r[4];
                __builtin_memcpy(d, __builtin_assume_aligned(X + pbo[b] + o, 4), 20);
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbit(d[i + 1], d[i], psh[b]);
                __builtin_memcpy(&f.b[b], r, 16);
            } else {
                __builtin_memcpy(&f.b[b], __builtin_assume_aligned(X + pbo[b] + o, 4), 16);
            }
        }
    };
    auto mma = [&](Frags& f) {
        const uint32_t k0 = f.last ? lm0 : ~0u, k1 = f.last ? lm1 : ~0u, k2 = f.last ? lm2 : ~0u,
                       k3 = f.last ? lm3 : ~0u;
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            uint4 u;
            __builtin_memcpy(&u, &f.b[b], 16);
            u.x &= k0;
            u.y &= k1;
            u.z &= k2;
            u.w &= k3;
            __builtin_memcpy(&f.b[b], &u, 16);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                acc[i][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[i], f.b[b], acc[i][b], 0, 0, 0);
        }
    };

    const int nk = a.S >> 1;   // K steps per stage (S is even)
    // sync: one buffer, each stage copied through registers after every wave
    // is done with the one before (no copy in flight during the MFMAs).
    const bool sync = a.sync;
    if (!sync) {
        issue(0, 0);
        gather(0, 0);
    }
    for (int s = 0; s < a.NS; ++s) {
        if (sync) {
            __syncthreads();   // every wave is done with the previous stage
            copy_stage(s, 0);
            gather(s, 0);
            __syncthreads();
        } else {
            // This wave's loads of stage s have landed, and (barrier) every
            // wave's, and every wave is done with stage s-1's buffer.
            wait_vm<0>();
            __syncthreads();
            if (s + 1 < a.NS) issue(s + 1, (s + 1) % kBufs); else issue_none();
            if (kPre && s + 1 < a.NS) gather_load(s + 1);
        }

        const unsigned char* A = smem + (size_t)(sync ? 0 : s % kBufs) * a.stage_bytes;
        const unsigned char* X = A + (size_t)a.S * 1024;
        Frags f0, f1;
        sms = hl < M ? hl : hl - M;
        soff = hl < M ? 16 * hl : xc2;
        fetch(f0, A, X, 0);
        int t = 0;
        for (; t + 2 <= nk; t += 2) {
            fetch(f1, A, X, t + 1);
            __builtin_amdgcn_sched_barrier(0);
            mma(f0);
            __builtin_amdgcn_sched_barrier(0);
            fetch(f0, A, X, t + 2);
            __builtin_amdgcn_sched_barrier(0);
            mma(f1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (t < nk) mma(f0);
        // The next stage's filter goes to the buffer freed by the barrier.
        if (!sync && s + 1 < a.NS) {
            if (kPre)
                gather_store(s + 1, (s + 1) % kBufs);
            else
                gather(s + 1, (s + 1) % kBufs);
        }
    }
    wait_vm<0>();

    // Output: lane holds pixel l32 of each block and channels
    // 8*(r/4) + 4*hl + r%4 of each 32-channel block. Blocks 2p and 2p+1 of a
    // wave are 64 consecutive pixels: swapping lanes 32-63 of the first with
    // lanes 0-31 of the second (v_permlane32_swap) gives one register with
    // channel cu for all 64 pixels and one with channel cu+4, so every store
    // writes 256 contiguous bytes of one channel plane.
    const __amdgpu_buffer_rsrc_t yb = raw_rsrc(y, a.ybytes);
    const bool all_co = co0 + kCoT <= Co;
#pragma unroll
    for (int p = 0; p < kNB / 2; ++p) {
        const int64_t qa = q0 + (wave * kNB + 2 * p) * 32 + lane;
        const bool ok = qa < qend;
        const int64_t q = ok ? qa : qend - 1;
        const int n = (int)a.divPlane.div((uint32_t)q);
        const int64_t pp = q - (int64_t)n * plane;
        const uint32_t vo = (uint32_t)((((int64_t)n * Co) * plane + pp) * 4);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int cu = co0 + i * 32 + 8 * (r >> 2) + (r & 3);
                const auto sv = __builtin_amdgcn_permlane32_swap(
                    __float_as_uint(acc[i][2 * p][r]), __float_as_uint(acc[i][2 * p + 1][r]), false,
                    false);
                if (ok && (all_co || cu < Co))
                    __builtin_amdgcn_raw_buffer_store_b32(sv[0], yb, (int)vo, (int)(cu * plane * 4), 0);
                if (ok && (all_co || cu + 4 < Co))
                    __builtin_amdgcn_raw_buffer_store_b32(sv[1], yb, (int)vo,
                                                          (int)((cu + 4) * plane * 4), 0);
            }
    }
}

constexpr int kDmax[] = {4, 6, 8, 10, 12, 16};

// Plans a launch; false if the shape is outside the kernel's envelope: packed
// rows a multiple of 8 elements
// (16-byte aligned regions), a stage of two channels in LDS, tiles touching
// at most kMaxSeg images, tensors addressable with 32-bit buffer offsets.
bool plan(const ConvShape& c, WsArgs& a, int& nwv, int& dmax)
{
    a.c = c;
    a.L = c.Wi * c.Hf;
    a.step = c.sw * c.Hf;
    if (a.L % 8 != 0) return false;
    a.M = ceil_div(c.Hf * c.Wf, 8);
    a.total = (int64_t)c.N * c.Ho * c.Wo;
    const int64_t plane = (int64_t)c.Ho * c.Wo;
    if (a.total >= 0x7fffffff || (int64_t)c.Ho * a.L >= 0x7fffffff) return false;
    bool found = false;
    for (int v : {8, 4}) {
        a.P = 32 * kNB * v;
        const int rows_max = (int)std::min<int64_t>((a.P - 1 + c.Wo - 1) / c.Wo + 1, (int64_t)c.N * c.Ho);
        a.kmax = (int)std::min<int64_t>(c.N - 1, (a.P - 1) / plane + 1);
        if (a.kmax + 1 > kMaxSeg) continue;
        // Halves of a channel region: the windows of P consecutive pixels
        // (row breaks add L - Wo*sw*Hf each when positive), the last window's
        // tail, and 8-element rounding per segment.
        const int64_t gap = std::max<int64_t>(0, (int64_t)a.L - (int64_t)c.Wo * a.step);
        const int64_t xc = (int64_t)(rows_max - 1) * gap + (int64_t)(a.P - 1) * a.step +
                           (int64_t)(a.kmax + 1) * (c.Hf * c.Wf + 16);
        a.XC = (int)((xc + 7) / 8 * 8);
        for (int cg : {4, 2}) {
            if (c.Ci % cg != 0 || (cg * a.M) % 2 != 0) continue;
            const int S = cg * a.M;
            const int NX = (int)ceil_div((int64_t)cg * a.XC * 2, 1024);
            const int need = ceil_div(NX, v);
            int dm = 0;
            for (int d : kDmax)
                if (d >= need) {
                    dm = d;
                    break;
                }
            if (!dm) continue;
            const int64_t stage = (int64_t)(S + NX) * 1024;
            const int64_t lds = kBufs * stage + 1024 + kSlack;   // slack: reads past a stage
            if (lds > kWsLds) continue;
            a.Cg = cg;
            a.S = S;
            a.NX = NX;
            a.stage_bytes = (uint32_t)stage;
            a.dummy = (uint32_t)(kBufs * stage);
            a.lds_bytes = (uint32_t)lds;
            nwv = v;
            dmax = dm;
            found = true;
            break;
        }
        if (found) break;
    }
    if (!found) return false;
    a.NS = c.Ci / a.Cg;
    a.co_tiles = ceil_div(c.Co, kCoT);
    a.px_tiles = (a.total + a.P - 1) / a.P;
    if (a.px_tiles * a.co_tiles > 0x7fffffff) return false;
    const int64_t wb = (int64_t)c.N * c.Ci * c.Ho * a.L * 2;
    const int64_t yb = (int64_t)c.N * c.Co * plane * 4;
    const int64_t wo = (int64_t)c.Co * c.Ci * c.Hf * c.Wf * 2;
    if (wb >= 0x7fffffff || yb >= (int64_t)kMiss || wo >= 0x7fffffff) return false;
    a.wsbytes = (uint32_t)wb;
    a.ybytes = (uint32_t)yb;
    a.worig = (uint32_t)wo;
    const int valid = c.Hf * c.Wf - 8 * (a.M - 1);   // real positions in a channel's last slice
    for (int d = 0; d < 4; ++d) {
        uint32_t m = 0;
        if (2 * d < valid) m |= 0xFFFFu;
        if (2 * d + 1 < valid) m |= 0xFFFF0000u;
        a.lastmask[d] = m;
    }
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divHo = FastDiv((uint32_t)c.Ho);
    a.divPlane = FastDiv((uint32_t)plane);
    a.swz = knob(KNOB_TILE_ORDER) != 1;
    a.sync = knob(KNOB_SYNC_STAGING) == 1;
    return true;
}

template <int NWV, int DMAX>
int launch_t(const uint16_t* ws, const uint16_t* w, float* y, const WsArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.px_tiles * a.co_tiles)), block(64 * NWV);
    if (a.step % 2) {
        ensure_lds_limit((const void*)conv_f16_ws_kernel<NWV, DMAX, true>, kWsLds);
        hipLaunchKernelGGL((conv_f16_ws_kernel<NWV, DMAX, true>), grid, block, a.lds_bytes, stream,
                           ws, w, y, a);
    } else {
        ensure_lds_limit((const void*)conv_f16_ws_kernel<NWV, DMAX, false>, kWsLds);
        hipLaunchKernelGGL((conv_f16_ws_kernel<NWV, DMAX, false>), grid, block, a.lds_bytes, stream,
                           ws, w, y, a);
    }
    return launch_status();
}

template <int NWV>
int launch_d(int dmax, const uint16_t* ws, const uint16_t* w, float* y, const WsArgs& a,
             hipStream_t stream)
{
    switch (dmax) {
    case 4: return launch_t<NWV, 4>(ws, w, y, a, stream);
    case 6: return launch_t<NWV, 6>(ws, w, y, a, stream);
    case 8: return launch_t<NWV, 8>(ws, w, y, a, stream);
    case 10: return launch_t<NWV, 10>(ws, w, y, a, stream);
    case 12: return launch_t<NWV, 12>(ws, w, y, a, stream);
    case 16: return launch_t<NWV, 16>(ws, w, y, a, stream);
    }
    return -1;
}

}  // namespace

bool f16_ws_applies(const ConvShape& c)
{
    WsArgs a;
    int nwv, dmax;
    return knob(KNOB_F16_WS) >= 0 && plan(c, a, nwv, dmax);
}

int launch_conv_f16_ws(const uint16_t* ws, const uint16_t* w, float* y, const ConvShape& c,
                       hipStream_t stream)
{
    WsArgs a;
    int nwv, dmax;
    if (knob(KNOB_F16_WS) < 0 || !plan(c, a, nwv, dmax)) return -1;
    if ((uintptr_t)ws % 16 != 0) return -1;
    return nwv == 8 ? launch_d<8>(dmax, ws, w, y, a, stream) : launch_d<4>(dmax, ws, w, y, a, stream);
}

}  // namespace im2win
