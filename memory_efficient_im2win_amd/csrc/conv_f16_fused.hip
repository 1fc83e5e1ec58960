// Fused fp16 im2win convolution on the CDNA4 matrix cores (fp32 accumulate).
//
// The half-precision path of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract: half
// precision multiply-accumulate on matrix hardware) for one MI355X. The
// contraction over Ci*Hf*Wf runs on v_mfma_f32_32x32x16_f16:
//
//  * GEMM view: rows = output channels (A = filters), columns = output
//    pixels (B = windows), K = (channel group g of 8, window tap j, channel
//    in the group). Pixels are numbered over the whole batch,
//    q = (n*Ho + ho)*Wo + wo. A workgroup of WCO x WPX waves owns
//    64*WCO channels and P = 32*NB*WPX consecutive pixels; each wave owns a
//    64-channel x 32*NB-pixel block (2 x NB MFMA tiles, AGPR accumulators).
//  * Per channel group the workgroup stages in LDS the window tile of its
//    pixels: the Hf input rows of each im2win row it needs, channel-
//    interleaved (16-byte entry = 8 channels of one input pixel), each input
//    row stored once even where the im2win rows of consecutive output rows
//    overlap (sh < Hf). Output rows of different images get separate rows.
//    Within a row the columns are stored stride-phase major, so the window
//    of a pixel is Hf x Wf entries at fixed offsets from its tap (0, 0), the
//    32 pixels of an MFMA block read 32 consecutive entries for every tap,
//    and every lane's 8-element K slice of B is one 16-byte LDS read.
//  * The filters of the group are staged as entries (tap j, channel co) in
//    the same K order, from the caller's prepacked copy when a workspace is
//    given (contiguous 16-byte loads) or gathered from w otherwise.
//  * The next group's global loads are issued into registers before the
//    MFMAs of the current group and written to LDS after them, so HBM/L2
//    latency overlaps the matrix work.
//  * One MFMA consumes two taps (j = 2t for lanes 0-31, 2t+1 for 32-63); an
//    odd tap count gets a zero filter entry and a zeroed B slice, so an
//    infinity next to a window never turns into NaN.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "knobs.hpp"

namespace im2win {

namespace {

constexpr int kMaxLds = 160 * 1024;
constexpr int kCoPad = kF16CoPad;   // prepacked filter: channels padded to a multiple of this

struct FusedArgs {
    ConvShape c;
    int P, co_tile, co_tiles;
    int64_t px_tiles, total;
    int rows_max, kmax, dup, RIN;   // output rows per tile, image breaks, sh<Hf overlap, LDS rows
    int HW, HWp, CG, Copad;
    int NU, RS;                     // columns per stride phase ceil(Wi/sw); entries per LDS row sw*NU
    int xentries;                   // LDS entries of the input rows: RIN * RS
    int xunits;                     // staging units: RIN * Wi / 2 (paired) or RIN * Wi
    bool xpair;                     // Wi even: rows fetched 2 columns x 8 channels at a time
    bool aligned;                   // tiles never cross images (kmax = 0)
    int64_t tiles_per_image;        // aligned tiling: ceil(Ho*Wo / P)
    int NWH, HPH;                   // filter stages per channel group, tap pairs per stage
    int KT;                         // entries of the tap offset table
    uint32_t xbytes, ybytes;        // sizes of x and y (each below 4 GiB: buffer addressing)
    FastDiv divWo, divHo, divWi, divHalfW, divS;
    bool swz;                       // XCD-grouped tile order
    bool sync;                      // next stage loaded after this one's MFMAs
};

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi)
{
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Buffer resources (raw_rsrc) cover [base, base + bytes): loads at
// soffset + voffset >= bytes return 0, which the kernel uses instead
// of per-lane branches; every load that can miss has soffset 0 and voffset
// kNoOff, which is out of range for any buffer the planner accepts.
constexpr uint32_t kNoOff = 0xFFFFFFF0u;

// Filters of channel group g as 16-byte entries (tap j, channel co):
// wpk[(g*HWp + j)*Copad + co] = w[co][8g..8g+7][j], zero beyond Co, Ci, HW.
// A workgroup packs channels co0 .. co0+3 of group g: for each channel the
// 8*HW elements w[co][8g..8g+7][0..HW) are contiguous in w, so they are read
// in order into LDS and each entry's 8 taps are gathered from there.
constexpr int kPackCo = 4;
__global__ __launch_bounds__(256) void f16_filter_pack_kernel(const uint16_t* __restrict__ w,
                                                              uint4* __restrict__ wpk,
                                                              FusedArgs a)
{
    extern __shared__ uint16_t fs[];   // [kPackCo][8 * HW]
    const int g = blockIdx.y, co0 = blockIdx.x * kPackCo;
    const int HW = a.HW, Ci = a.c.Ci, Co = a.c.Co;
    const int nc = min(8, Ci - 8 * g);
    const int per = 8 * HW;
    // Sixteen independent loads per thread in flight at a time.
    for (int i0 = 0; i0 < kPackCo * per; i0 += 16 * 256) {
        uint16_t v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int i = i0 + k * 256 + threadIdx.x;
            const int col = i / per, r = i - col * per;   // r = q*HW + j
            const int co = co0 + col;
            v[k] = i < kPackCo * per && co < Co && r < nc * HW
                       ? w[((int64_t)co * Ci + 8 * g) * HW + r]
                       : (uint16_t)0;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int i = i0 + k * 256 + threadIdx.x;
            if (i < kPackCo * per) fs[i] = v[k];
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kPackCo * a.HWp; i += 256) {
        const int j = i / kPackCo, col = i - j * kPackCo;
        uint32_t v[4] = {0, 0, 0, 0};
        if (j < HW) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                v[q >> 1] |= (uint32_t)fs[col * per + q * HW + j] << (16 * (q & 1));
        }
        wpk[((int64_t)g * a.HWp + j) * a.Copad + co0 + col] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// The same entries, one thread each, gathered straight from w (filters with
// more than 256 taps).
__global__ __launch_bounds__(256) void f16_filter_gather_kernel(const uint16_t* __restrict__ w,
                                                                uint4* __restrict__ wpk,
                                                                FusedArgs a)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)a.CG * a.HWp * a.Copad;
    if (e >= total) return;
    const int co = (int)(e % a.Copad);
    const int64_t gj = e / a.Copad;
    const int j = (int)(gj % a.HWp), g = (int)(gj / a.HWp);
    uint16_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (co < a.c.Co && j < a.HW) {
        const uint16_t* src = w + ((int64_t)co * a.c.Ci + 8 * g) * a.HW + j;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (8 * g + q < a.c.Ci) v[q] = src[(int64_t)q * a.HW];
    }
    wpk[e] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]),
                        pack2(v[6], v[7]));
}

// Per-thread staging capacities (checked by the planner).
constexpr int kXUnits = 6;    // input units of 2 columns x 8 channels (paired path)
constexpr int kXEnt = 12;     // input entries (gather path)
constexpr int kWEnt = 8;      // filter entries
constexpr int kWSlack = 4;    // spare filter-entry rows (reads one pair past a stage)

// LDS bytes of a launch: input rows, filter entries (+ slack), tap table.
size_t fused_lds_bytes(int xentries, int HPH, int co_tile, int KT)
{
    return ((size_t)xentries + (size_t)(2 * HPH + kWSlack) * co_tile) * 16 +
           ((size_t)KT * 4 + 15) / 16 * 16;
}

// LDS layout of one staged input row: column c is entry (c % sw)*NU + c / sw
// (column-stride-phase major), so the 32 pixels of an MFMA block, whose
// window columns are wo*sw + kw, read 32 consecutive entries for every tap.
template <int WCO, int WPX, int NB, bool XPAIR, bool WPK>
__global__ __launch_bounds__(64 * WCO * WPX) void conv_f16_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint4* __restrict__ wpk, float* __restrict__ y, FusedArgs a)
{
    constexpr int NT = 64 * WCO * WPX;
    constexpr int COT = 64 * WCO;

    extern __shared__ __align__(16) uint4 lds[];
    uint4* X = lds;
    uint4* Wl = lds + a.xentries;

    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co;
    const int sh = a.c.sh, sw = a.c.sw;
    const int Ho = a.c.Ho, Wo = a.c.Wo, Hf = a.c.Hf, Wf = a.c.Wf;
    const int HW = a.HW, HWp = a.HWp, RS = a.RS, NU = a.NU;

    // XCD-grouped tile order unless the tile_order knob asks for launch order.
    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x, a.swz);
    const int co_t = (int)(bid % a.co_tiles);
    const int64_t pt = bid / a.co_tiles;
    const int co0 = co_t * COT;
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
    const int wco = wave % WCO, wpx = wave / WCO;

    // Entry of tap (0, 0) of each pixel: LDS row of its output row gr
    // (tile-relative r = gr - gr0, image k: r*sh + k*dup) times RS, plus wo.
    int xb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        int64_t q = q0 + (wpx * NB + b) * 32 + l32;
        if (q >= qend) q = qend - 1;
        const int gr = (int)a.divWo.div((uint32_t)(q - (int64_t)gr0 * Wo)) + gr0;
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int k = (int)a.divHo.div((uint32_t)gr) - n0;
        xb[b] = ((gr - gr0) * sh + k * a.dup) * RS + wo;
    }
    // A entry of this lane for tap pair 0: tap hl, channel column wco*64 + l32.
    const int abase = hl * COT + wco * 64 + l32;

    floatx16_t acc[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][b][r] = 0.f;

    // LDS row i -> (image n, input row h); false if no input row maps there.
    // Segment k holds the output rows of image n0+k that fall in the tile.
    auto x_src = [&](int i, int& n, int& h) -> bool {
        for (int k = 0; k <= a.kmax; ++k) {
            const int nk = n0 + k;
            const int first = max(gr0, nk * Ho), last = min(grl, nk * Ho + Ho - 1);
            if (first > last) break;
            const int S = (first - gr0) * sh + k * a.dup;
            const int span = (last - first) * sh + Hf;
            if (i >= S && i < S + span) {
                n = nk;
                h = (first - nk * Ho) * sh + (i - S);
                return true;
            }
        }
        return false;
    };
    auto col_entry = [&](int c) {
        const int u = (int)a.divS.div((uint32_t)c);
        return (c - u * sw) * NU + u;
    };

    // ---- staging: global -> registers (group g) -> LDS --------------------------
    // Paired path: a unit is 2 consecutive columns of one LDS row, fetched as
    // 8 channels x 4 bytes and split into 2 entries. Where a unit reads from
    // and writes to does not depend on the channel group, so it is worked out
    // once: a byte offset from channel 0 of image 0 (the channel plane is a
    // uniform base per load) and two LDS entries.
    constexpr int NXU = XPAIR ? kXUnits : kXEnt;
    uint32_t xp[XPAIR ? kXUnits * 8 : 1];
    uint4 xg[XPAIR ? 1 : kXEnt];
    uint4 wv[kWEnt];
    uint32_t uoff[NXU];          // source byte offset from channel 0 (kNoOff: no source)
    int udst0[NXU], udst1[NXU];  // LDS entries (udst0 < 0: unit not staged)
    const int hcols = Wi >> 1;
    const int64_t cstride = (int64_t)Hi * Wi;
#pragma unroll
    for (int u = 0; u < NXU; ++u) {
        const int e = tid + u * NT;
        udst0[u] = udst1[u] = -1;
        uoff[u] = kNoOff;
        if (e < a.xunits) {
            int i, col;
            if (XPAIR) {
                i = (int)a.divHalfW.div((uint32_t)e);
                col = 2 * (e - i * hcols);
                udst1[u] = i * RS + col_entry(col + 1);
            } else {
                i = (int)a.divWi.div((uint32_t)e);
                col = e - i * Wi;
            }
            udst0[u] = i * RS + col_entry(col);
            int n, h;
            if (x_src(i, n, h))
                uoff[u] = (uint32_t)(((((int64_t)n * Ci) * Hi + h) * Wi + col) * 2);
        }
    }
    // Filter entries of a stage: byte offsets from the stage's first tap.
    const int wstage = 2 * a.HPH * COT;   // filter entries per stage
    uint32_t woff[kWEnt];
#pragma unroll
    for (int u = 0; u < kWEnt; ++u) {
        const int e = tid + u * NT;
        const int jj = e / COT, col = e - (e / COT) * COT;
        if (WPK)
            woff[u] = e < wstage ? (uint32_t)((jj * a.Copad + co0 + col) * 16) : kNoOff;
        else
            woff[u] = e < wstage && co0 + col < Co
                          ? (uint32_t)((((int64_t)(co0 + col) * Ci) * HW + jj) * 2)
                          : kNoOff;
    }

    // Stage st = (channel group g, filter part h): the input rows of group g
    // are staged with part 0; part h holds taps [2*h*HPH, 2*(h+1)*HPH).
    // Loads the filter part of stage st and, if with_x, the input rows of
    // channel group gx (into registers).
    auto load_stage = [&](int st, bool with_x, int gx) {
        const int g = st / a.NWH, h = st - (st / a.NWH) * a.NWH;
        const int cb = 8 * g;     // channel group of the filter part
        if (with_x) {
            const int cbx = 8 * gx;   // channel group of the input rows
            // One buffer per channel plane; a missing channel gets an empty buffer.
            __amdgpu_buffer_rsrc_t pl[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int64_t first = (int64_t)(cbx + q) * cstride * 2;
                pl[q] = raw_rsrc(x + (int64_t)(cbx + q < Ci ? cbx + q : 0) * cstride,
                                 cbx + q < Ci ? (uint32_t)(a.xbytes - first) : 0u);
            }
#pragma unroll
            for (int u = 0; u < NXU; ++u) {
                if (XPAIR) {
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        xp[u * 8 + q] = __builtin_amdgcn_raw_buffer_load_b32(pl[q], (int)uoff[u], 0, 0);
                } else {
                    uint32_t v[4] = {0, 0, 0, 0};
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        if (cbx + q < Ci)
                            v[q >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                             pl[q], (int)uoff[u], 0, 0)
                                         << (16 * (q & 1));
                    xg[u] = make_uint4(v[0], v[1], v[2], v[3]);
                }
            }
        }
        const int j0 = 2 * h * a.HPH;
        if (WPK) {
            // Taps j0 .. HWp-1 of group g; entries past HWp read as zero.
            const __amdgpu_buffer_rsrc_t wb =
                raw_rsrc(wpk + ((int64_t)g * HWp + j0) * a.Copad, (uint32_t)((HWp - j0) * a.Copad * 16));
#pragma unroll
            for (int u = 0; u < kWEnt; ++u) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(wb, (int)woff[u], 0, 0);
                wv[u] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        } else {
            // Gather from w: tap j0 + jj of channel cb + q is (q*HW + j0)*2 bytes
            // past the entry's offset; missing taps and channels read as zero.
            const __amdgpu_buffer_rsrc_t wb =
                raw_rsrc(w, (uint32_t)((int64_t)Co * Ci * HW * 2));
#pragma unroll
            for (int u = 0; u < kWEnt; ++u) {
                const int jj = (tid + u * NT) / COT;
                const bool ok = j0 + jj < HW && woff[u] != kNoOff;
                uint32_t v[4] = {0, 0, 0, 0};
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (cb + q < Ci)
                        v[q >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                         wb,
                                         (int)(ok ? woff[u] + (uint32_t)(((cb + q) * HW + j0) * 2)
                                                  : kNoOff),
                                         0, 0)
                                     << (16 * (q & 1));
                wv[u] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        }
    };
    auto store_stage = [&](bool with_x) {
        if (with_x) {
#pragma unroll
            for (int u = 0; u < NXU; ++u) {
                if (udst0[u] < 0) continue;
                if (XPAIR) {
                    const uint32_t* d = &xp[u * 8];   // d[c]: channel c, columns col (lo), col+1 (hi)
                    uint4 lo, hi;
                    lo.x = (d[0] & 0xffffu) | (d[1] << 16);
                    lo.y = (d[2] & 0xffffu) | (d[3] << 16);
                    lo.z = (d[4] & 0xffffu) | (d[5] << 16);
                    lo.w = (d[6] & 0xffffu) | (d[7] << 16);
                    hi.x = (d[0] >> 16) | (d[1] & 0xffff0000u);
                    hi.y = (d[2] >> 16) | (d[3] & 0xffff0000u);
                    hi.z = (d[4] >> 16) | (d[5] & 0xffff0000u);
                    hi.w = (d[6] >> 16) | (d[7] & 0xffff0000u);
                    X[udst0[u]] = lo;
                    X[udst1[u]] = hi;
                } else {
                    X[udst0[u]] = xg[u];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kWEnt; ++u) {
            const int e = tid + u * NT;
            if (e < wstage) Wl[e] = wv[u];
        }
    };

    // Window offsets of the taps in filter order j = kh*Wf + kw (from the
    // pixel's tap (0, 0): kh*RS + (kw % sw)*NU + kw / sw), tabulated once per
    // workgroup so each lane reads its own tap's offset (one LDS read per
    // pair, two pairs ahead) instead of walking taps on the scalar unit.
    // Entries from HW on repeat tap HW-1 (in range; such reads are unused
    // or zeroed).
    int* T = reinterpret_cast<int*>(Wl + (2 * a.HPH + kWSlack) * COT);
    for (int j = tid; j < a.KT; j += NT) {
        const int jj = j < HW ? j : HW - 1;
        const int kh = jj / Wf, kw = jj - (jj / Wf) * Wf;
        T[j] = kh * RS + (kw % sw) * NU + kw / sw;
    }
    // Fragments of one tap pair: A for the two 32-channel blocks, B for the
    // NB pixel blocks. Pair t holds taps 2t (lanes 0-31) and 2t+1 (32-63);
    // on0, on1 hold the window offsets of this lane's taps of pairs t, t+1.
    struct Frags {
        half8_t a[2], b[NB];
    };
    int on0 = 0, on1 = 0;
    auto fetch = [&](Frags& f, int t, int tl) {
        const int o = on0;
        on0 = on1;
        on1 = T[2 * t + 4 + hl];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 u = Wl[abase + 2 * tl * COT + i * 32];
            __builtin_memcpy(&f.a[i], &u, 16);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint4 u = X[xb[b] + o];
            __builtin_memcpy(&f.b[b], &u, 16);
        }
    };
    auto mma = [&](const Frags& f) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                acc[i][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[i], f.b[b], acc[i][b], 0, 0, 0);
    };

    const int nfull = HW >> 1;          // tap pairs with two real taps
    const bool odd = (HW & 1) != 0;

    const int npairs = nfull + (odd ? 1 : 0);
    const int nstages = a.CG * a.NWH;

    // The input rows of group g+1 are fetched during the first filter part
    // of group g (NWH >= 2: two or more stages ahead, more latency covered)
    // and written to LDS after its last part.
    load_stage(0, true, 0);
    store_stage(true);
    __syncthreads();
    for (int st = 0; st < nstages; ++st) {
        const int g = st / a.NWH, h = st % a.NWH;
        const bool xnext = a.NWH >= 2 ? h == 0 && g + 1 < a.CG : st + 1 < nstages;
        // sync: the next stage's loads wait until this stage's MFMAs are
        // issued, so no copy is in flight while they run.
        if (!a.sync && st + 1 < nstages) load_stage(st + 1, xnext, g + 1);

        // Pairs [t0, t1) of this stage; the fragments of pair t+1 are read
        // from LDS while the MFMAs of pair t run. The loop body fetches
        // unconditionally (one pair past the stage at most: in-allocation
        // reads that are never used), so every path into an MFMA has the
        // same reads outstanding.
        const int t0 = h * a.HPH, t1 = min(npairs, t0 + a.HPH);
        const int tf = min(t1, nfull);
        const bool pad = odd && t1 > nfull;   // this stage ends with tap HW-1 alone
        Frags f0, f1;
        on0 = T[2 * t0 + hl];
        on1 = T[2 * t0 + 2 + hl];
        fetch(f0, t0, 0);
        int t = t0;
        for (; t + 2 <= tf; t += 2) {
            fetch(f1, t + 1, t + 1 - t0);
            __builtin_amdgcn_sched_barrier(0);
            mma(f0);
            __builtin_amdgcn_sched_barrier(0);
            fetch(f0, t + 2, t + 2 - t0);
            __builtin_amdgcn_sched_barrier(0);
            mma(f1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Left: f0 = pair t.
        if (t < tf) {
            mma(f0);
            if (pad) fetch(f0, nfull, nfull - t0);
            ++t;
        }
        if (pad) {
            // Last tap with a zero partner: the filter entry of tap HW is zero
            // and lanes 32-63 zero their B slice (so Inf/NaN cannot leak in).
            const uint32_t keep = hl ? 0u : ~0u;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                uint4 u;
                __builtin_memcpy(&u, &f0.b[b], 16);
                u.x &= keep; u.y &= keep; u.z &= keep; u.w &= keep;
                __builtin_memcpy(&f0.b[b], &u, 16);
            }
            mma(f0);
        }

        if (st + 1 < nstages) {
            __syncthreads();
            if (a.sync) load_stage(st + 1, xnext, g + 1);
            store_stage((st + 1) % a.NWH == 0);
            __syncthreads();
        }
    }

    // Output: lane holds pixel l32 of each block and channels
    // 8*(r/4) + 4*hl + r%4 of each 32-channel block. Blocks 2p and 2p+1 of a
    // wave are 64 consecutive pixels: swapping lanes 32-63 of the first with
    // lanes 0-31 of the second (v_permlane32_swap) gives one register with
    // channel cu for all 64 pixels and one with channel cu+4, so every store
    // writes 256 contiguous bytes of one channel plane.
    static_assert(NB % 2 == 0, "blocks are stored in pairs");
    const int64_t plane = (int64_t)Ho * Wo;
    const __amdgpu_buffer_rsrc_t yb = raw_rsrc(y, a.ybytes);
    const bool all_co = co0 + COT <= Co;
#pragma unroll
    for (int p = 0; p < NB / 2; ++p) {
        const int64_t qa = q0 + (wpx * NB + 2 * p) * 32 + lane;
        const bool ok = qa < qend;
        const int64_t q = ok ? qa : qend - 1;
        const int gr = (int)(q / Wo);
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int n = (int)a.divHo.div((uint32_t)gr), ho = gr - n * Ho;
        const uint32_t voff = (uint32_t)((((int64_t)n * Co) * plane + (int64_t)ho * Wo + wo) * 4);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int cu = co0 + wco * 64 + i * 32 + 8 * (r >> 2) + (r & 3);
                const auto sv = __builtin_amdgcn_permlane32_swap(
                    __float_as_uint(acc[i][2 * p][r]), __float_as_uint(acc[i][2 * p + 1][r]), false,
                    false);
                if (ok && (all_co || cu < Co))
                    __builtin_amdgcn_raw_buffer_store_b32(sv[0], yb, (int)voff, (int)(cu * plane * 4),
                                                          0);
                if (ok && (all_co || cu + 4 < Co))
                    __builtin_amdgcn_raw_buffer_store_b32(sv[1], yb, (int)voff,
                                                          (int)((cu + 4) * plane * 4), 0);
            }
    }
}

// Plans the fused launch; returns false if the shape is outside its envelope.
// KNOB_F16_WPX / KNOB_F16_NWH override the waves along pixels and the filter
// stages per channel group (tuning and tests only). One 64-channel column of
// waves (WCO = 1).
bool plan(const ConvShape& c, FusedArgs& a, int& wco, int& wpx, int& nb)
{
    a.c = c;
    a.HW = c.Hf * c.Wf;
    a.HWp = (a.HW + 1) & ~1;
    a.CG = ceil_div(c.Ci, 8);
    a.KT = (a.HWp + 8 + 3) & ~3;   // reads reach tap index 2*(HWp/2) + 5
    a.Copad = ceil_div(c.Co, kCoPad) * kCoPad;
    a.total = (int64_t)c.N * c.Ho * c.Wo;
    a.dup = std::max(0, c.Hf - c.sh);
    if ((int64_t)c.N * c.Ho > 0x7fffffff) return false;
    nb = 2;
    wco = 1;
    a.xpair = c.Wi % 2 == 0;
    a.NU = ceil_div(c.Wi, c.sw);
    a.RS = c.sw * a.NU;
    const int npairs = a.HWp / 2;
    const int64_t plane = (int64_t)c.Ho * c.Wo;
    // Smallest workgroup LDS first: two workgroups of four waves per CU let one
    // stage its next channel group while the other runs MFMAs.
    bool found = false;
    const int env_wpx = knob(KNOB_F16_WPX), env_nwh = knob(KNOB_F16_NWH);
    for (int budget : {80 * 1024, kMaxLds}) {
        for (wpx = 8; wpx >= 1; wpx /= 2) {
            if (env_wpx ? wpx != env_wpx : wpx == 8) continue;
            a.co_tile = 64 * wco;
            a.P = 32 * nb * wpx;
            a.rows_max = (a.P - 1) / c.Wo + 2;
            a.tiles_per_image = (plane + a.P - 1) / a.P;
            a.aligned = (double)(a.tiles_per_image * a.P) <= 1.05 * (double)plane;
            a.kmax = a.aligned || a.rows_max <= 1 ? 0 : ceil_div(a.rows_max - 1, c.Ho);
            a.RIN = (a.rows_max - 1) * c.sh + c.Hf + a.kmax * a.dup;
            a.xentries = a.RIN * a.RS;
            a.xunits = a.xpair ? a.RIN * (c.Wi / 2) : a.RIN * c.Wi;
            const int nt = 64 * wco * wpx;
            if (a.xunits > (a.xpair ? kXUnits : kXEnt) * nt) continue;
            for (a.NWH = 1; a.NWH <= npairs; ++a.NWH) {
                if (env_nwh && a.NWH < std::min(env_nwh, npairs)) continue;
                a.HPH = ceil_div(npairs, a.NWH);
                const int wentries = 2 * a.HPH * a.co_tile;
                const int64_t bytes =
                    (int64_t)fused_lds_bytes(a.xentries, a.HPH, a.co_tile, a.KT);
                if (bytes <= budget && wentries <= kWEnt * nt) {
                    found = true;
                    break;
                }
            }
            if (found) break;
        }
        if (found) break;
    }
    if (!found) return false;
    if (a.aligned) a.kmax = 0;
    // Buffer addressing: x, y and the prepacked filter each below 4 GiB.
    const int64_t xb = (int64_t)c.N * c.Ci * c.Hi * c.Wi * 2;
    const int64_t yb = (int64_t)c.N * c.Co * c.Ho * c.Wo * 4;
    const int64_t wb = (int64_t)a.CG * a.HWp * a.Copad * 16;
    if (xb >= (int64_t)kNoOff || yb >= (int64_t)kNoOff || wb >= (int64_t)kNoOff) return false;
    a.xbytes = (uint32_t)xb;
    a.ybytes = (uint32_t)yb;
    a.co_tiles = ceil_div(c.Co, a.co_tile);
    a.px_tiles = a.aligned ? (int64_t)c.N * a.tiles_per_image : (a.total + a.P - 1) / a.P;
    if (a.px_tiles * a.co_tiles > 0x7fffffff) return false;
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divHo = FastDiv((uint32_t)c.Ho);
    a.divWi = FastDiv((uint32_t)c.Wi);
    a.divHalfW = FastDiv((uint32_t)std::max(1, c.Wi / 2));
    a.divS = FastDiv((uint32_t)c.sw);
    a.swz = knob(KNOB_TILE_ORDER) != 1;
    a.sync = knob(KNOB_SYNC_STAGING) == 1;
    return true;
}

template <int WCO, int WPX, int NB, bool XVEC, bool WPK>
int launch_t(const uint16_t* x, const uint16_t* w, const uint4* wpk, float* y,
             const FusedArgs& a, hipStream_t stream)
{
    ensure_lds_limit((const void*)conv_f16_fused_kernel<WCO, WPX, NB, XVEC, WPK>, kMaxLds);
    const size_t lds = fused_lds_bytes(a.xentries, a.HPH, a.co_tile, a.KT);
    hipLaunchKernelGGL((conv_f16_fused_kernel<WCO, WPX, NB, XVEC, WPK>),
                       dim3((unsigned)(a.px_tiles * a.co_tiles)), dim3(64 * WCO * WPX), lds,
                       stream, x, w, wpk, y, a);
    return launch_status();
}

template <int WCO, int WPX>
int launch_w(const uint16_t* x, const uint16_t* w, const uint4* wpk, float* y,
             const FusedArgs& a, hipStream_t stream)
{
    if (a.xpair)
        return wpk ? launch_t<WCO, WPX, 2, true, true>(x, w, wpk, y, a, stream)
                   : launch_t<WCO, WPX, 2, true, false>(x, w, wpk, y, a, stream);
    return wpk ? launch_t<WCO, WPX, 2, false, true>(x, w, wpk, y, a, stream)
               : launch_t<WCO, WPX, 2, false, false>(x, w, wpk, y, a, stream);
}

}  // namespace

// Which kernel a fused fp16 call runs on: the row-staged kernel for the
// shapes it takes (x 16-byte aligned), then the thin-layer kernel, then the
// wide-tile kernel, then the channel-interleaved kernel above; 0 if none
// takes the shape. The filter, prepacked or gathered, follows the kernel's
// layout.
enum F16Route { kRouteNone = 0, kRouteReuse, kRouteRows, kRouteThin, kRouteWide, kRouteFused };

F16Route f16_route(const ConvShape& c, const void* x)
{
    if (f16_reuse_applies(c) && (uintptr_t)x % 16 == 0) return kRouteReuse;
    if (f16_rows_applies(c) && (uintptr_t)x % 16 == 0) return kRouteRows;
    if (f16_thin_applies(c)) return kRouteThin;
    if (f16_wide_applies(c, kCoPad)) return kRouteWide;
    FusedArgs a;
    int wco, wpx, nb;
    return plan(c, a, wco, wpx, nb) ? kRouteFused : kRouteNone;
}

size_t f16_filter_pack_bytes(const ConvShape& c)
{
    // Enough for whichever layout the planners pick, whatever the knobs: the
    // channel-interleaved entries of this kernel and the wide-tile one, or
    // the (channel, filter row) slices of the row-staged and thin-layer ones.
    size_t b = (size_t)ceil_div(c.Ci, 8) * (size_t)((c.Hf * c.Wf + 1) & ~1) *
               (size_t)(ceil_div(c.Co, kCoPad) * kCoPad) * 16;
    if (c.Wf <= 8 && c.Hf * c.Wf <= 256) b = std::max(b, f16_slices_filter_bytes(c));
    return b;
}

const char* f16_fused_kernel_name(const ConvShape& c, const void* x, bool prepacked)
{
    const F16Route r = f16_route(c, x);
    if ((r == kRouteWide || r == kRouteFused) && prepacked && f16_res_applies(c, kCoPad, x, x))
        return "conv_f16_res_kernel";
    switch (r) {
    case kRouteReuse: return "conv_f16_reuse_kernel";
    case kRouteRows: return "conv_f16_rows_kernel";
    case kRouteThin: return "conv_f16_thin_kernel";
    case kRouteWide: return "conv_f16_wide_kernel";
    case kRouteFused: return "conv_f16_fused_kernel";
    default: return "conv_generic_kernel";
    }
}

int launch_f16_filter_pack(const uint16_t* w, void* wpk, const ConvShape& c, const void* x,
                           hipStream_t stream)
{
    const F16Route r = f16_route(c, x);
    if (r == kRouteNone) return -1;
    if (r == kRouteRows || r == kRouteReuse) return launch_f16_rows_filter_pack(w, wpk, c, stream);
    if (r == kRouteThin) return launch_f16_slices_filter_pack(w, wpk, c, stream);
    return launch_f16_interleaved_filter_pack(w, wpk, c, stream);
}

size_t f16_interleaved_filter_bytes(const ConvShape& c)
{
    return (size_t)ceil_div(c.Ci, 8) * (size_t)((c.Hf * c.Wf + 1) & ~1) *
           (size_t)(ceil_div(c.Co, kCoPad) * kCoPad) * 16;
}

int launch_f16_interleaved_filter_pack(const uint16_t* w, void* wpk, const ConvShape& c,
                                       hipStream_t stream)
{
    FusedArgs a{};
    a.c = c;
    a.HW = c.Hf * c.Wf;
    a.HWp = (a.HW + 1) & ~1;
    a.CG = ceil_div(c.Ci, 8);
    a.Copad = ceil_div(c.Co, kCoPad) * kCoPad;
    // LDS of one workgroup: kPackCo channels x 8 x HW taps (HW <= 256: 16 KB).
    const size_t lds = (size_t)kPackCo * 8 * a.HW * 2;
    if (a.HW <= 256 && a.CG <= 65535) {
        hipLaunchKernelGGL(f16_filter_pack_kernel,
                           dim3((unsigned)(a.Copad / kPackCo), (unsigned)a.CG), dim3(256), lds,
                           stream, w, (uint4*)wpk, a);
        return launch_status();
    }
    const int64_t total = (int64_t)a.CG * a.HWp * a.Copad;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return -1;
    hipLaunchKernelGGL(f16_filter_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w,
                       (uint4*)wpk, a);
    return launch_status();
}

int launch_conv_f16_fused(const uint16_t* x, const uint16_t* w, const void* wpk, float* y,
                          const ConvShape& c, hipStream_t stream)
{
    const F16Route r = f16_route(c, x);
    if (r == kRouteNone) return -1;
    if (r == kRouteReuse) return launch_conv_f16_reuse(x, wpk, w, y, c, stream);
    if (r == kRouteRows) return launch_conv_f16_rows(x, wpk, w, y, c, stream);
    if (r == kRouteThin) return launch_conv_f16_thin(x, wpk, w, y, c, stream);
    if (wpk && f16_res_applies(c, kCoPad, x, y))
        return launch_conv_f16_res(x, wpk, y, c, kCoPad, false, stream);
    if (r == kRouteWide) return launch_conv_f16_wide(x, wpk, w, y, c, kCoPad, stream);
    FusedArgs a;
    int wco, wpx, nb;
    if (!plan(c, a, wco, wpx, nb)) return -1;
    const uint4* wp = static_cast<const uint4*>(wpk);
    if (wco == 1 && wpx == 8) return launch_w<1, 8>(x, w, wp, y, a, stream);
    if (wco == 1 && wpx == 4) return launch_w<1, 4>(x, w, wp, y, a, stream);
    if (wco == 1 && wpx == 2) return launch_w<1, 2>(x, w, wp, y, a, stream);
    if (wco == 1 && wpx == 1) return launch_w<1, 1>(x, w, wp, y, a, stream);
    return -1;
}

}  // namespace im2win
