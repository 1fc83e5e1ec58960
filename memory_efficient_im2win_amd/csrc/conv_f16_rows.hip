// fp16 im2win convolution on the CDNA4 matrix cores, with the input rows
// copied to LDS by direct global-to-LDS loads.
//
// The half-precision path of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract:
// half-precision multiply-accumulate on matrix hardware), laid out for the
// im2win property of "Im2win: Memory Efficient Convolution On SIMD
// Architectures" (Abstract): the part of a window that lies in one input row
// is one contiguous run of that row.
//
//  * GEMM view: rows = output channels (A = filters), columns = output
//    pixels numbered over the batch (B = windows), K = (input channel c,
//    filter row kh, filter column kw), with kw padded to 8. One K slice of 8
//    is one (c, kh): for a pixel it is the 8 consecutive input columns
//    wo*sw .. wo*sw+7 of input row ho*sh+kh, so each lane's B operand of
//    v_mfma_f32_32x32x16_f16 is one 16-byte LDS read. Lanes 0-31 take slice
//    2t, lanes 32-63 slice 2t+1. Filter taps kw >= Wf are zero in the
//    prepacked filter and the matching B halves are masked to zero, so an
//    infinity just outside a window never turns into NaN.
//  * A workgroup owns 64 output channels (two 32-row blocks) and
//    P = 128 * NWV consecutive pixels; each wave owns 128 pixels (four
//    32-column blocks): a 2 x 4 register tile of accumulators, so every A
//    read feeds four MFMAs and every B read two.
//  * A stage is Cg input channels. Its filter slices (prepacked as
//    [c][kh][co][8 halves], one kilobyte per slice and channel tile) and the
//    input rows its pixels cover (copied as they lie in x, one LDS row per
//    (channel, input row)) are fetched with buffer_load_dwordx4 ... lds: no
//    registers, no transposition. Three stage buffers rotate; the loads of
//    stage s+2 are issued as stage s starts, and one barrier per stage both
//    publishes stage s and frees the buffer of stage s-1. Without a
//    prepacked filter the slices of stage s+2 are gathered from w instead
//    (loaded as stage s starts, written after its MFMAs); there two buffers
//    (loads one stage ahead) are used when they let a stage hold twice the
//    channels, which halves the gather rounds.
//  * The loads are issued from inline assembly so that the compiler, which
//    would otherwise wait for every outstanding LDS load before each LDS
//    read, leaves the pipelining to the explicit waits here.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "knobs.hpp"

namespace im2win {

namespace {

constexpr int kRowsLds = 160 * 1024;
constexpr int kCoT = 64;                  // output channels per tile
constexpr int kNB = 4;                    // 32-pixel blocks per wave
constexpr int kBufsMax = 3;               // stage buffers (3: loads two stages ahead; 2: one)
constexpr int kSlack = 2048;              // LDS past the last buffer: reads one pair past a stage
constexpr uint32_t kMiss = 0xFFFFFFF0u;   // vector offset past every accepted buffer
constexpr int kGL = 16;                   // most dword gather loads per thread and stage

struct RowsArgs {
    ConvShape c;
    int P, co_tiles;
    int64_t px_tiles, total, tiles_per_image;
    bool aligned;                   // tiles never cross images
    int rows_max, kmax, dup, RIN;   // output rows per tile, image breaks, sh<Hf overlap, LDS rows per channel
    int RP;                         // halves per LDS row (multiple of 8)
    int Cg, S, NX, NS, Copad;       // channels per stage, slices per stage (Cg*Hf), row kilobytes
                                    // per stage, stages (Ci/Cg), prepacked filter channels
    uint32_t stage_bytes;           // (S + NX) KB: filter slices, then rows
    int bufs;                       // stage buffers: loads run bufs - 1 stages ahead
    uint32_t dummy;                 // LDS byte offset of the landing kilobyte of unused loads
    uint32_t lds_bytes;
    uint32_t xbytes, ybytes, wbytes, worig;   // x, y, prepacked filter, filter in w's layout
    uint32_t mask[4];               // B dwords: halves kw >= Wf cleared
    // Dword filter gather (no prepacked filter, w 4-byte aligned): gl dword
    // loads per thread and stage (0: one 16-byte entry per thread and load
    // round instead); RD dwords of w per output channel and stage, wco bytes
    // between output channels; a thread's dword index advances by gjs*RD + grs
    // per load; wfm = ceil(2^16 / Wf).
    int gl, gjs, grs;
    uint32_t RD, wco, wfm;
    bool swz;                       // XCD-grouped tile order
    bool sync;                      // stages copied through registers, one buffer
    FastDiv divWo, divHo;
};




// Filter slices (c, kh) as 16-byte entries of the 8 taps kw of one output
// channel: wp[(c*Hf + kh)*Copad + co] = w[co][c][kh][0..7], zero for kw >= Wf
// and co >= Co. A workgroup packs channels co0 .. co0+3 and input channels
// c0 .. c0+7: for each output channel those input channels' Hf*Wf taps are
// contiguous in w, so they are read in order into LDS and each entry's taps
// are gathered from there.
constexpr int kPackCo = 4;
__global__ __launch_bounds__(256) void f16_rows_filter_pack_kernel(const uint16_t* __restrict__ w,
                                                                   uint4* __restrict__ wp,
                                                                   RowsArgs a)
{
    extern __shared__ uint16_t fs[];   // [kPackCo][8 * Hf * Wf]
    const int Ci = a.c.Ci, Co = a.c.Co, Hf = a.c.Hf, Wf = a.c.Wf;
    const int co0 = blockIdx.x * kPackCo, c0 = 8 * blockIdx.y;
    const int nc = min(8, Ci - c0);
    const int per = 8 * Hf * Wf;
    // Sixteen independent loads per thread in flight at a time.
    for (int i0 = 0; i0 < kPackCo * per; i0 += 16 * 256) {
        uint16_t v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int i = i0 + k * 256 + threadIdx.x;
            const int col = i / per, r = i - col * per;   // r = (c - c0)*Hf*Wf + kh*Wf + kw
            const int co = co0 + col;
            v[k] = i < kPackCo * per && co < Co && r < nc * Hf * Wf
                       ? w[((int64_t)co * Ci + c0) * Hf * Wf + r]
                       : (uint16_t)0;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int i = i0 + k * 256 + threadIdx.x;
            if (i < kPackCo * per) fs[i] = v[k];
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kPackCo * nc * Hf; i += 256) {
        const int ck = i / kPackCo, col = i - ck * kPackCo;   // ck = (c - c0)*Hf + kh
        uint32_t v[4] = {0, 0, 0, 0};
        for (int kw = 0; kw < Wf; ++kw)
            v[kw >> 1] |= (uint32_t)fs[col * per + ck * Wf + kw] << (16 * (kw & 1));
        wp[((int64_t)c0 * Hf + ck) * a.Copad + co0 + col] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// WPK: the filter slices come prepacked (wp) by direct loads; otherwise each
// stage's slices are gathered from w, two stages ahead, after a stage's
// MFMAs (its direct-load slots then land in the dummy kilobyte, so every
// wave still issues DMAX loads per stage).
template <int NWV, int DMAX, bool M3, bool WPK>
__global__ __launch_bounds__(64 * NWV) void conv_f16_rows_kernel(const uint16_t* __restrict__ x,
                                                                 const uint4* __restrict__ wp,
                                                                 const uint16_t* __restrict__ w,
                                                                 float* __restrict__ y, RowsArgs a)
{
    constexpr int NT = 64 * NWV;
    extern __shared__ __align__(16) unsigned char smem[];
    const uint32_t lbase =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co;
    const int sh = a.c.sh, sw = a.c.sw;
    const int Ho = a.c.Ho, Wo = a.c.Wo, Hf = a.c.Hf;

    // XCD-grouped tile order unless the tile_order knob asks for launch order.
    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x, a.swz);
    const int co_t = (int)(bid % a.co_tiles);
    const int64_t pt = bid / a.co_tiles;
    const int co0 = co_t * kCoT;
    int64_t q0, qend;
    if (a.aligned) {   // tile pt = (image, tile within the image)
        const int64_t img = pt / a.tiles_per_image;
        const int64_t plane = (int64_t)Ho * Wo;
        q0 = img * plane + (pt - img * a.tiles_per_image) * a.P;
        qend = min(q0 + a.P, (img + 1) * plane);
    } else {
        q0 = pt * a.P;
        qend = q0 + a.P < a.total ? q0 + a.P : a.total;
    }
    const int gr0 = (int)(q0 / Wo);
    const int grl = (int)((qend - 1) / Wo);
    const int n0 = (int)a.divHo.div((uint32_t)gr0);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int wave = uniform(tid >> 6);

    // Byte offset, within a stage's rows, of each pixel's tap (c=0, kh=0,
    // kw=0): LDS row of its output row gr (tile-relative r*sh plus image
    // breaks k*dup) times the row pitch, plus its first column wo*sw.
    int pb[kNB];
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
        int64_t q = q0 + (wave * kNB + b) * 32 + l32;
        if (q >= qend) q = qend - 1;
        const int gr = (int)a.divWo.div((uint32_t)(q - (int64_t)gr0 * Wo)) + gr0;
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int k = (int)a.divHo.div((uint32_t)gr) - n0;
        pb[b] = (((gr - gr0) * sh + k * a.dup) * a.RP + wo * sw) * 2;
    }

    // LDS row i -> (image n, input row h); false if no input row maps there.
    // Segment k holds the output rows of image n0+k that fall in the tile.
    auto x_src = [&](int i, int& n, int& h) -> bool {
        for (int k = 0; k <= a.kmax; ++k) {
            const int nk = n0 + k;
            const int first = max(gr0, nk * Ho), last = min(grl, nk * Ho + Ho - 1);
            if (first > last) break;
            const int S0 = (first - gr0) * sh + k * a.dup;
            const int span = (last - first) * sh + Hf;
            if (i >= S0 && i < S0 + span) {
                n = nk;
                h = (first - nk * Ho) * sh + (i - S0);
                return true;
            }
        }
        return false;
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
            int n, h;
            if (cl < a.Cg && 8 * cc < Wi && x_src(r, n, h))
                v = (uint32_t)(((((int64_t)n * Ci + cl) * Hi + h) * Wi + 8 * cc) * 2);
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

    floatx16_t acc[2][kNB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int b = 0; b < kNB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][b][r] = 0.f;

    struct Frags {
        half8_t a[2], b[kNB];
    };
    const uint32_t m0 = a.mask[0], m1 = a.mask[1], m2 = a.mask[2], m3 = a.mask[3];
    const int abase = hl * kCoT + l32;   // A entry of slice hl, channel l32
    // This lane's slice 2t + hl = (channel cl, filter row kh) sits at byte
    // (cl*RIN + kh)*RP*2 from a pixel's tap (0, 0, 0) within the stage's
    // rows. It advances by two slices per pair, carrying kh into cl.
    const int rp2 = a.RP * 2, wrap = (a.RIN - Hf) * a.RP * 2;
    int skh = 0, soff = 0;
    auto fetch = [&](Frags& f, const unsigned char* A, const unsigned char* X, int t) {
        const int o = soff;
        skh += 2;
        soff += 2 * rp2;
        if (skh >= Hf) { skh -= Hf; soff += wrap; }
        if (skh >= Hf) { skh -= Hf; soff += wrap; }
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_memcpy(&f.a[i], A + (size_t)(abase + 2 * t * kCoT + i * 32) * 16, 16);
        // B addresses are 4-byte aligned (even column stride, row pitch a
        // multiple of 8 halves) but not 16-byte aligned; stated so, the reads
        // become aligned dword-pair reads instead of the much slower
        // unaligned 16-byte form.
#pragma unroll
        for (int b = 0; b < kNB; ++b)
            __builtin_memcpy(&f.b[b], __builtin_assume_aligned(X + pb[b] + o, 4), 16);
    };
    // The padded taps are masked here, just before the MFMAs, not at the
    // read: a mask at the read would wait for that read before the previous
    // pair's MFMAs could issue. With Wf >= 6 (M3) only the last dword holds
    // padded taps.
    auto mma = [&](Frags& f) {
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            uint4 u;
            __builtin_memcpy(&u, &f.b[b], 16);
            if (!M3) {
                u.x &= m0;
                u.y &= m1;
                u.z &= m2;
            }
            u.w &= m3;
            __builtin_memcpy(&f.b[b], &u, 16);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                acc[i][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[i], f.b[b], acc[i][b], 0, 0, 0);
        }
    };

    // Without a prepacked filter: entry (slice m, channel co0 + j) of stage
    // sg holds the taps of w[co0 + j][sg*Cg + m/Hf][m%Hf][*] (zeros past Wf
    // and Co).
    auto gather = [&](int sg, int sb) {
        const __amdgpu_buffer_rsrc_t rw = raw_rsrc(w, a.worig);
        uint4* F = reinterpret_cast<uint4*>(smem + (size_t)sb * a.stage_bytes);
        const int ne = a.S * 64;
        for (int e0 = 0; e0 < ne; e0 += 2 * NT) {
            uint32_t hv[2][8];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int e = e0 + k * NT + tid;
                const int m = e >> 6, co = co0 + (e & 63);
                const int c = sg * a.Cg + m / Hf, kh = m - (m / Hf) * Hf;
                const uint32_t src = e < ne && co < Co
                                         ? (uint32_t)((((co * Ci + c) * Hf + kh) * a.c.Wf) * 2)
                                         : kMiss;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    hv[k][q] = __builtin_amdgcn_raw_buffer_load_b16(
                        rw, (int)(q < a.c.Wf ? src + 2 * q : kMiss), 0, 0);
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int e = e0 + k * NT + tid;
                if (e < ne)
                    F[e] = make_uint4(hv[k][0] | (hv[k][1] << 16), hv[k][2] | (hv[k][3] << 16),
                                      hv[k][4] | (hv[k][5] << 16), hv[k][6] | (hv[k][7] << 16));
            }
        }
    };

    // Dword gather: for its 64 channels a stage's taps are 64 runs of RD
    // dwords in w (channel co0+j, input channels sg*Cg.., all Hf*Wf taps),
    // read with consecutive threads on consecutive dwords of a run. Each of
    // a dword's two halves goes to the entry of its slice (tap t of the run
    // is slice t / Wf, column t % Wf). The loads of stage s+D (D: stages the
    // loads run ahead) go out with stage s's direct loads and are written to
    // LDS after its MFMAs.
    // Channels past Co fall outside w's range and read zeros; halves
    // kw >= Wf of every entry are zeroed once below and never written again.
    uint32_t gv[kGL];
    const int gj0 = tid / (int)a.RD, gq0 = tid - gj0 * (int)a.RD;
    auto gather_load = [&](int sg) {
        const __amdgpu_buffer_rsrc_t rw = raw_rsrc(w, a.worig);
        const uint32_t base = (uint32_t)co0 * a.wco + (uint32_t)sg * a.RD * 4;
        int j = gj0, r = gq0;
        // Opaque per call: the offsets do not depend on the stage, and
        // hoisting them out of the stage loop would cost 3*kGL registers.
        asm volatile("" : "+v"(j), "+v"(r));
#pragma unroll
        for (int i = 0; i < kGL; ++i) {
            if (i < a.gl) {
                const uint32_t src = j < 64 ? base + (uint32_t)j * a.wco + (uint32_t)r * 4 : kMiss;
                gv[i] = __builtin_amdgcn_raw_buffer_load_b32(rw, (int)src, 0, 0);
            }
            j += a.gjs;
            r += a.grs;
            if (r >= (int)a.RD) {
                r -= (int)a.RD;
                ++j;
            }
        }
    };
    auto gather_store = [&](int sb) {
        uint16_t* F = reinterpret_cast<uint16_t*>(smem + (size_t)sb * a.stage_bytes);
        int j = gj0, r = gq0;
        asm volatile("" : "+v"(j), "+v"(r));
#pragma unroll
        for (int i = 0; i < kGL; ++i) {
            if (i < a.gl && j < 64) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t t = 2 * (uint32_t)r + h;
                    const uint32_t m = (t * a.wfm) >> 16;
                    const uint32_t kw = t - m * (uint32_t)a.c.Wf;
                    F[((m * 64 + j) << 3) + kw] = (uint16_t)(gv[i] >> (16 * h));
                }
            }
            j += a.gjs;
            r += a.grs;
            if (r >= (int)a.RD) {
                r -= (int)a.RD;
                ++j;
            }
        }
    };
    const bool coal = !WPK && a.gl > 0;
    if (coal && a.c.Wf < 8) {
        for (int e = tid; e < a.bufs * a.S * 64; e += NT) {
            const int b = e / (a.S * 64);
            uint16_t* F = reinterpret_cast<uint16_t*>(smem + (size_t)b * a.stage_bytes);
            const int el = e - b * a.S * 64;
            for (int kw = a.c.Wf; kw < 8; ++kw) F[el * 8 + kw] = 0;
        }
    }

    const int nk = a.S >> 1;   // K steps per stage (S is even)
    const int D = a.bufs - 1;  // stages the loads run ahead (2 or 1)
    // sync: one buffer, each stage copied through registers after every wave
    // is done with the one before, and computed once it has landed (no copy
    // in flight during the MFMAs).
    const bool sync = a.sync;
    if (!sync) {
        issue(0, 0);
        if (D == 2) {
            if (a.NS > 1) issue(1, 1); else issue_none();
        }
        if (coal) {
            gather_load(0);
            gather_store(0);
            if (D == 2 && a.NS > 1) {
                gather_load(1);
                gather_store(1);
            }
        } else if (!WPK) {
            gather(0, 0);
            if (D == 2 && a.NS > 1) gather(1, 1);
        }
    }
    for (int s = 0; s < a.NS; ++s) {
        if (sync) {
            __syncthreads();   // every wave is done with the previous stage
            copy_stage(s, 0);
            if (coal) {
                gather_load(s);
                gather_store(0);
            } else if (!WPK) {
                gather(s, 0);
            }
            __syncthreads();
        } else {
            // This wave's loads of stage s have landed (those of stage s+1
            // may still be in flight with three buffers).
            if (D == 2)
                wait_vm<DMAX>();
            else
                wait_vm<0>();
            __syncthreads();      // every wave's; and stage s-1's buffer is free
            if (s + D < a.NS) issue(s + D, (s + D) % a.bufs); else issue_none();
            if (coal && s + D < a.NS) gather_load(s + D);
        }

        const unsigned char* A = smem + (size_t)(sync ? 0 : s % a.bufs) * a.stage_bytes;
        const unsigned char* X = A + (size_t)a.S * 1024;
        Frags f0, f1;
        skh = hl < Hf ? hl : hl - Hf;       // slice hl (Hf = 1: channel 1, row 0)
        soff = hl < Hf ? hl * rp2 : a.RIN * rp2;
        fetch(f0, A, X, 0);
        // The fragments of pair t+1 are read while the MFMAs of pair t run.
        // Reads are unconditional (the last ones fall one pair past the
        // stage, inside the allocation, and are never used), so every path
        // into an MFMA has the same reads outstanding and the waits stay
        // exact.
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
        // Stage s+D's buffer was freed by the barrier above.
        if (!sync && !WPK && s + D < a.NS) {
            if (coal)
                gather_store((s + D) % a.bufs);
            else
                gather(s + D, (s + D) % a.bufs);
        }
    }
    wait_vm<0>();   // the last (unused) loads have landed before the workgroup ends

    // Output: lane holds pixel l32 of each block and channels
    // 8*(r/4) + 4*hl + r%4 of each 32-channel block. Blocks 2p and 2p+1 of a
    // wave are 64 consecutive pixels: swapping lanes 32-63 of the first with
    // lanes 0-31 of the second (v_permlane32_swap) gives one register with
    // channel cu for all 64 pixels and one with channel cu+4, so every store
    // writes 256 contiguous bytes of one channel plane (32-pixel stores into
    // two planes made the HBM writes about 1.3x the output).
    const int64_t plane = (int64_t)Ho * Wo;
    const __amdgpu_buffer_rsrc_t yb = raw_rsrc(y, a.ybytes);
    const bool all_co = co0 + kCoT <= Co;
#pragma unroll
    for (int p = 0; p < kNB / 2; ++p) {
        const int64_t qa = q0 + (wave * kNB + 2 * p) * 32 + lane;
        const bool ok = qa < qend;
        const int64_t q = ok ? qa : qend - 1;
        const int gr = (int)(q / Wo);
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int n = (int)a.divHo.div((uint32_t)gr), ho = gr - n * Ho;
        const uint32_t vo = (uint32_t)((((int64_t)n * Co) * plane + (int64_t)ho * Wo + wo) * 4);
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

// Load instructions per wave and stage the kernel is built for.
constexpr int kDmax[] = {4, 5, 6, 8, 12, 16};

// Plans a launch; false if the shape is outside the kernel's envelope:
// even column stride, Wf <= 8, Hf*Wf <= 256 (the filter pack's LDS), Wi a
// multiple of 8 (16-byte row chunks),
// Ci a multiple of the stage's channel count, tensors addressable with
// 32-bit buffer offsets. Knobs (tuning and tests): KNOB_F16_ROWS < 0 turns
// the kernel off, KNOB_F16_ROWS_NWV picks the waves per workgroup,
// KNOB_TILE_ORDER = 1 keeps tiles in launch order and KNOB_F16_ROWS_BUFS =
// 2 or 3 fixes the stage buffers. bufs_want: stage buffers to plan for (0:
// three, or the knob).
bool plan(const ConvShape& c, RowsArgs& a, int& nwv, int& dmax, int bufs_want = 0)
{
    if (knob(KNOB_F16_ROWS) < 0) return false;
    if (c.Wf > 8 || c.sw % 2 != 0 || c.Wi % 8 != 0 || c.Hf * c.Wf > 256) return false;
    a.c = c;
    a.total = (int64_t)c.N * c.Ho * c.Wo;
    a.dup = std::max(0, c.Hf - c.sh);
    a.RP = ((std::max(c.Wi, (c.Wo - 1) * c.sw + 8) + 7) / 8) * 8;
    a.Copad = ceil_div(c.Co, kCoT) * kCoT;
    if ((int64_t)c.N * c.Ho > 0x7fffffff) return false;
    const int64_t plane = (int64_t)c.Ho * c.Wo;
    const int env_nwv = knob(KNOB_F16_ROWS_NWV);
    const int env_bufs = knob(KNOB_F16_ROWS_BUFS);
    const int bufs = env_bufs == 2 || env_bufs == 3 ? env_bufs : bufs_want == 2 ? 2 : kBufsMax;
    bool found = false;
    for (int v : {8, 4}) {
        if (env_nwv && v != env_nwv) continue;
        a.P = 32 * kNB * v;
        // Output rows a tile touches (never more than the batch has) and
        // image breaks inside a tile (never more than N - 1).
        a.rows_max = (int)std::min<int64_t>((a.P - 1) / c.Wo + 2, (int64_t)c.N * c.Ho);
        a.tiles_per_image = (plane + a.P - 1) / a.P;
        a.aligned = (double)(a.tiles_per_image * a.P) <= 1.05 * (double)plane;
        a.kmax = a.aligned || a.rows_max <= 1 ? 0
                                              : std::min(c.N - 1, ceil_div(a.rows_max - 1, c.Ho));
        a.RIN = (a.rows_max - 1) * c.sh + c.Hf + a.kmax * a.dup;
        for (int cg : {4, 2}) {
            if (c.Ci % cg != 0 || (cg * c.Hf) % 2 != 0) continue;
            const int S = cg * c.Hf;
            const int NX = (int)ceil_div(cg * a.RIN * a.RP * 2, 1024);
            const int need = ceil_div(S + NX, v);
            int dm = 0;
            for (int d : kDmax)
                if (d >= need) {
                    dm = d;
                    break;
                }
            if (!dm) continue;
            const int64_t stage = (int64_t)(S + NX) * 1024;
            const int64_t lds = bufs * stage + 1024 + kSlack;
            if (lds > kRowsLds) continue;
            a.Cg = cg;
            a.S = S;
            a.NX = NX;
            a.stage_bytes = (uint32_t)stage;
            a.dummy = (uint32_t)(bufs * stage);
            a.bufs = bufs;
            a.lds_bytes = (uint32_t)lds;
            nwv = v;
            dmax = dm;
            found = true;
            break;
        }
        if (found) break;
    }
    if (!found) return false;
    if (a.aligned) a.kmax = 0;
    a.NS = c.Ci / a.Cg;
    a.co_tiles = ceil_div(c.Co, kCoT);
    a.px_tiles = a.aligned ? (int64_t)c.N * a.tiles_per_image : (a.total + a.P - 1) / a.P;
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
    a.divHo = FastDiv((uint32_t)c.Ho);
    a.swz = knob(KNOB_TILE_ORDER) != 1;
    a.sync = knob(KNOB_SYNC_STAGING) == 1;
    return true;
}

template <int NWV, int DMAX, bool M3, bool WPK>
int launch_t(const uint16_t* x, const uint4* wp, const uint16_t* w, float* y, const RowsArgs& a,
             hipStream_t stream)
{
    ensure_lds_limit((const void*)conv_f16_rows_kernel<NWV, DMAX, M3, WPK>, kRowsLds);
    hipLaunchKernelGGL((conv_f16_rows_kernel<NWV, DMAX, M3, WPK>),
                       dim3((unsigned)(a.px_tiles * a.co_tiles)), dim3(64 * NWV), a.lds_bytes,
                       stream, x, wp, w, y, a);
    return launch_status();
}

template <int NWV, bool M3, bool WPK>
int launch_d(int dmax, const uint16_t* x, const uint4* wp, const uint16_t* w, float* y,
             const RowsArgs& a, hipStream_t stream)
{
    switch (dmax) {
    case 4: return launch_t<NWV, 4, M3, WPK>(x, wp, w, y, a, stream);
    case 5: return launch_t<NWV, 5, M3, WPK>(x, wp, w, y, a, stream);
    case 6: return launch_t<NWV, 6, M3, WPK>(x, wp, w, y, a, stream);
    case 8: return launch_t<NWV, 8, M3, WPK>(x, wp, w, y, a, stream);
    case 12: return launch_t<NWV, 12, M3, WPK>(x, wp, w, y, a, stream);
    case 16: return launch_t<NWV, 16, M3, WPK>(x, wp, w, y, a, stream);
    }
    return -1;
}

template <bool WPK>
int launch_p(int nwv, int dmax, const uint16_t* x, const uint4* wp, const uint16_t* w, float* y,
             const RowsArgs& a, hipStream_t stream)
{
    if (nwv == 8 && a.c.Wf >= 6) return launch_d<8, true, WPK>(dmax, x, wp, w, y, a, stream);
    if (nwv == 8) return launch_d<8, false, WPK>(dmax, x, wp, w, y, a, stream);
    return launch_d<4, false, WPK>(dmax, x, wp, w, y, a, stream);
}

}  // namespace

bool f16_rows_applies(const ConvShape& c)
{
    RowsArgs a;
    int nwv, dmax;
    return plan(c, a, nwv, dmax);
}

size_t f16_rows_filter_bytes(const ConvShape& c)
{
    RowsArgs a;
    int nwv, dmax;
    if (!plan(c, a, nwv, dmax)) return 0;
    return (size_t)a.wbytes;
}

int launch_f16_rows_filter_pack(const uint16_t* w, void* wp, const ConvShape& c, hipStream_t stream)
{
    RowsArgs a;
    int nwv, dmax;
    if (!plan(c, a, nwv, dmax)) return -1;
    return launch_f16_slices_filter_pack(w, wp, c, stream);
}

size_t f16_slices_filter_bytes(const ConvShape& c)
{
    return (size_t)c.Ci * c.Hf * (size_t)(ceil_div(c.Co, kCoT) * kCoT) * 16;
}

int launch_f16_slices_filter_pack(const uint16_t* w, void* wp, const ConvShape& c,
                                  hipStream_t stream)
{
    if (c.Wf > 8 || c.Hf * c.Wf > 256 || ceil_div(c.Ci, 8) > 65535) return -1;
    RowsArgs a{};
    a.c = c;
    a.Copad = ceil_div(c.Co, kCoT) * kCoT;
    // LDS of one workgroup: kPackCo channels x 8 input channels x Hf*Wf taps
    // (at most 16 KB).
    const size_t lds = (size_t)kPackCo * 8 * c.Hf * c.Wf * 2;
    hipLaunchKernelGGL(f16_rows_filter_pack_kernel,
                       dim3((unsigned)(a.Copad / kPackCo), (unsigned)ceil_div(c.Ci, 8)), dim3(256),
                       lds, stream, w, static_cast<uint4*>(wp), a);
    return launch_status();
}

int launch_conv_f16_rows(const uint16_t* x, const void* wp, const uint16_t* w, float* y,
                         const ConvShape& c, hipStream_t stream)
{
    RowsArgs a;
    int nwv, dmax;
    if (!plan(c, a, nwv, dmax)) return -1;
    // Rows are fetched in 16-byte chunks from 16-byte boundaries.
    if ((uintptr_t)x % 16 != 0 || (uintptr_t)wp % 16 != 0) return -1;
    const uint4* w4 = static_cast<const uint4*>(wp);
    if (!w4) {
        // Gathering the filter costs a round of loads per stage: with two
        // buffers a stage may hold twice the channels (half the stages).
        RowsArgs a2;
        int nwv2, dmax2;
        if (plan(c, a2, nwv2, dmax2, 2) && a2.Cg > a.Cg) {
            a = a2;
            nwv = nwv2;
            dmax = dmax2;
        }
    }
    a.gl = a.gjs = a.grs = 0;
    a.RD = 1;
    a.wco = a.wfm = 0;
    if (!w4 && (uintptr_t)w % 4 == 0) {
        // S is even, so RD is whole; Ci is even, so every run starts on a dword.
        const int nt = 64 * nwv;
        const int rd = a.S * c.Wf / 2;
        const int gl = ceil_div(64 * rd, nt);
        const int64_t wco = (int64_t)c.Ci * c.Hf * c.Wf * 2;
        if (gl <= kGL && (int64_t)ceil_div(c.Co, kCoT) * kCoT * wco < (int64_t)kMiss) {
            a.gl = gl;
            a.RD = (uint32_t)rd;
            a.gjs = nt / rd;
            a.grs = nt % rd;
            a.wco = (uint32_t)wco;
            a.wfm = (uint32_t)ceil_div(65536, c.Wf);
        }
    }
    return w4 ? launch_p<true>(nwv, dmax, x, w4, w, y, a, stream)
              : launch_p<false>(nwv, dmax, x, w4, w, y, a, stream);
}

}  // namespace im2win
