// fp16 im2win convolution on the CDNA4 matrix cores for layers with many
// output channels (fp32 accumulate; filter prepacked or gathered).
//
// The half-precision path of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract: half
// precision multiply-accumulate on matrix hardware; Table I, cv5: 256
// filters of 96 x 5 x 5), built on the im2win rows of "Im2win: Memory
// Efficient Convolution On SIMD Architectures" (Abstract).
//
//  * GEMM view as in the channel-interleaved fused kernel: rows = output
//    channels (A = filters), columns = output pixels numbered over the batch
//    (B = windows), K = (channel group g of 8, window tap j, channel in the
//    group). The im2win rows of a tile sit in LDS channel-interleaved (one
//    16-byte entry = 8 channels of one input column, columns stride-phase
//    major), so every lane's 8-element K slice of A or B is one aligned
//    16-byte LDS read.
//  * A workgroup owns 128 output channels x 512 pixels. By default 8 waves
//    (two per SIMD) each hold all 128 channels x 64 pixels, a 4 x 2 tile of
//    32 x 32 accumulators, so each A read feeds two MFMAs and each B read
//    four (0.75 KB of LDS per MFMA); the alternative is 4 waves of 4 x 4
//    (256 accumulators, one wave per SIMD, 0.5 KB per MFMA).
//  * A stage is one channel group: the filter entries (tap, channel) of the
//    group for the tile's 128 channels, copied from the prepacked filter by
//    direct global-to-LDS loads (contiguous kilobytes, no registers) or,
//    without one, gathered from w after the previous group's MFMAs; and the
//    tile's input rows of the group, gathered through registers (8 channel
//    planes -> one entry). Two stage buffers alternate: the loads of group
//    g+1 are issued after the barrier that opens group g and land while its
//    MFMAs run; one barrier per group.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "knobs.hpp"

namespace im2win {

namespace {

constexpr int kWideLds = 160 * 1024;
constexpr int kCoW = 128;                 // output channels per tile (4 MFMA blocks)
constexpr int kPW = 512;                  // pixels per tile
constexpr int kXUW = 1024;                // paired staging units per tile
constexpr int kXEW = 1536;                // single-column staging entries per tile
constexpr int kSlackW = 8 * 1024;         // reads run up to two pairs past a stage
constexpr uint32_t kMissW = 0xFFFFFFF0u;  // vector offset past every accepted buffer

struct WideArgs {
    ConvShape c;
    int co_tiles;
    int64_t px_tiles, total, tiles_per_image;
    bool aligned;                   // tiles never cross images
    int rows_max, kmax, dup, RIN;   // output rows per tile, image breaks, sh<Hf overlap, LDS rows
    int HW, HWp, CG, Copad;
    int NU, RS;                     // columns per stride phase; entries per LDS row
    int xentries, xunits;           // LDS entries of the input rows; staging units
    int S;                          // filter kilobytes per stage (2 * HWp)
    int KT;                         // entries of the tap offset table
    uint32_t fbytes;                // filter part of a stage: HWp * 128 * 16
    uint32_t stage_bytes;           // filter part + input rows
    uint32_t tab;                   // LDS byte offset of the tap table
    uint32_t lds_bytes;
    uint32_t xbytes, ybytes, wbytes, worig;   // x, y, prepacked filter, filter in w's layout
    FastDiv divWo, divHo, divWi, divHalfW, divS;
    bool swz;                       // XCD-grouped tile order
    bool sync;                      // groups copied through registers, one buffer
};



// NW waves of NB 32-pixel blocks each (NW * NB * 32 = kPW). WPK: the filter
// comes prepacked (wpk); otherwise each stage gathers its entries from w.
template <int NW, int NB, bool XPAIR, bool WPK>
__global__ __launch_bounds__(64 * NW) void conv_f16_wide_kernel(const uint16_t* __restrict__ x,
                                                             const uint4* __restrict__ wpk,
                                                             const uint16_t* __restrict__ w,
                                                             float* __restrict__ y, WideArgs a)
{
    static_assert(NW * NB * 32 == kPW, "tile width");
    constexpr int kNBW = NB, kWavesW = NW, kNTW = 64 * NW;
    extern __shared__ __align__(16) unsigned char smem[];
    const uint32_t lbase =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co;
    const int sh = a.c.sh, sw = a.c.sw;
    const int Ho = a.c.Ho, Wo = a.c.Wo, Hf = a.c.Hf, Wf = a.c.Wf;
    const int HW = a.HW, RS = a.RS, NU = a.NU;

    // XCD-grouped tile order unless the tile_order knob asks for launch order.
    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x, a.swz);
    const int co_t = (int)(bid % a.co_tiles);
    const int64_t pt = bid / a.co_tiles;
    const int co0 = co_t * kCoW;
    int64_t q0, qend;
    if (a.aligned) {   // tile pt = (image, tile within the image)
        const int64_t img = pt / a.tiles_per_image;
        const int64_t plane = (int64_t)Ho * Wo;
        q0 = img * plane + (pt - img * a.tiles_per_image) * kPW;
        qend = min(q0 + kPW, (img + 1) * plane);
    } else {
        q0 = pt * kPW;
        qend = q0 + kPW < a.total ? q0 + kPW : a.total;
    }
    const int gr0 = (int)(q0 / Wo);
    const int grl = (int)((qend - 1) / Wo);
    const int n0 = (int)a.divHo.div((uint32_t)gr0);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int wave = uniform(tid >> 6);

    // Entry of tap (0, 0) of each pixel within a stage's input rows: LDS row
    // of its output row gr (tile-relative r*sh plus image breaks k*dup)
    // times RS, plus wo.
    int xb[kNBW];
#pragma unroll
    for (int b = 0; b < kNBW; ++b) {
        int64_t q = q0 + (wave * kNBW + b) * 32 + l32;
        if (q >= qend) q = qend - 1;
        const int gr = (int)a.divWo.div((uint32_t)(q - (int64_t)gr0 * Wo)) + gr0;
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int k = (int)a.divHo.div((uint32_t)gr) - n0;
        xb[b] = ((gr - gr0) * sh + k * a.dup) * RS + wo;
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
    auto col_entry = [&](int c) {
        const int u = (int)a.divS.div((uint32_t)c);
        return (c - u * sw) * NU + u;
    };

    // Input staging units (independent of the channel group): source byte
    // offset from channel 0 of image 0 (kMissW: no source row) and LDS
    // entries (udst0 < 0: not staged). Paired: 2 columns x 8 channels,
    // fetched as 8 dwords and split into 2 entries.
    constexpr int NXU = (XPAIR ? kXUW : kXEW) / kNTW;
    uint32_t uoff[NXU];
    int udst0[NXU], udst1[NXU];
    const int hcols = Wi >> 1;
#pragma unroll
    for (int u = 0; u < NXU; ++u) {
        const int e = tid + u * kNTW;
        udst0[u] = udst1[u] = -1;
        uoff[u] = kMissW;
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
    uint32_t xp[XPAIR ? kXUW * 8 : 1];
    uint4 xg[XPAIR ? 1 : kXEW];
    const int64_t cstride = (int64_t)Hi * Wi;

    auto load_x = [&](int g) {
        const int cb = 8 * g;
        __amdgpu_buffer_rsrc_t pl[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int64_t first = (int64_t)(cb + q) * cstride * 2;
            pl[q] = raw_rsrc(x + (int64_t)(cb + q < Ci ? cb + q : 0) * cstride,
                         cb + q < Ci ? (uint32_t)(a.xbytes - first) : 0u);
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
                    v[q >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(pl[q], (int)uoff[u],
                                                                                0, 0)
                                 << (16 * (q & 1));
                xg[u] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        }
    };
    auto store_x = [&](int sb) {
        uint4* X = reinterpret_cast<uint4*>(smem + (size_t)sb * a.stage_bytes + a.fbytes);
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
    };
    // Filter of channel group g: kilobyte m of the stage is tap m/2, channels
    // co0 + 64*(m%2) .. +63, i.e. entries (g*HWp + m/2)*Copad + co0 + 64*(m%2)
    // + lane of the prepacked filter. Wave v issues kilobytes v, v+4, ...
    auto dma_w = [&](int g, int sb) {
        const uint32_t go = (uint32_t)g * a.HWp * a.Copad * 16;
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(wpk + (int64_t)g * a.HWp * a.Copad, a.wbytes - go);
        const uint32_t dst = lbase + (uint32_t)sb * a.stage_bytes;
        const uint32_t lo = (uint32_t)(co0 + lane) * 16;
        for (int m = wave; m < a.S; m += kWavesW)
            lds_dma16(r, dst + (uint32_t)m * 1024,
                   lo + (uint32_t)(m >> 1) * a.Copad * 16 + (uint32_t)(m & 1) * 1024);
    };
    // The same kilobytes copied through registers (synchronous staging).
    auto copy_w = [&](int g, int sb) {
        const uint32_t go = (uint32_t)g * a.HWp * a.Copad * 16;
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(wpk + (int64_t)g * a.HWp * a.Copad, a.wbytes - go);
        unsigned char* dst = smem + (size_t)sb * a.stage_bytes + 16 * lane;
        const uint32_t lo = (uint32_t)(co0 + lane) * 16;
#pragma unroll 4
        for (int m = wave; m < a.S; m += kWavesW) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(
                r, (int)(lo + (uint32_t)(m >> 1) * a.Copad * 16 + (uint32_t)(m & 1) * 1024), 0, 0);
            *reinterpret_cast<uint4*>(dst + (size_t)m * 1024) = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    // Without a prepacked filter: half c of entry (tap j, channel co0 + k) is
    // w[co0 + k][8g + c][j] (zero past HW, Co, Ci). A thread takes the
    // (k, c) pairs tid, tid + NT, ... and their taps in chunks, written to
    // LDS as each chunk arrives.
    auto gather_w = [&](int g, int sb) {
        constexpr int NPR = 8 * kCoW / kNTW;   // (k, c) pairs per thread
        constexpr int JC = 32 / NPR;           // taps per chunk
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(w, a.worig);
        unsigned short* F = reinterpret_cast<unsigned short*>(smem + (size_t)sb * a.stage_bytes);
        uint32_t base[NPR];
        int dst[NPR];
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
            const int pr = tid + p * kNTW, k = pr >> 3, c = pr & 7;
            const int co = co0 + k, ch = 8 * g + c;
            base[p] = co < Co && ch < Ci ? (uint32_t)(((int64_t)co * Ci + ch) * HW * 2) : kMissW;
            dst[p] = k * 8 + c;
        }
        for (int j0 = 0; j0 < a.HWp; j0 += JC) {
            uint32_t v[NPR][JC];
#pragma unroll
            for (int p = 0; p < NPR; ++p)
#pragma unroll
                for (int q = 0; q < JC; ++q) {
                    const int j = j0 + q;
                    v[p][q] = __builtin_amdgcn_raw_buffer_load_b16(
                        r, (int)(j < HW && base[p] != kMissW ? base[p] + 2 * j : kMissW), 0, 0);
                }
#pragma unroll
            for (int p = 0; p < NPR; ++p)
#pragma unroll
                for (int q = 0; q < JC; ++q)
                    if (j0 + q < a.HWp) F[(j0 + q) * kCoW * 8 + dst[p]] = (unsigned short)v[p][q];
        }
    };

    // The same entries with each pair's run of taps read as whole dwords:
    // the HW taps of w[co0 + k][8g + c][*] are one run of w, read from the
    // dword boundary at or below it with four 16-byte loads (all issued
    // before any is used; up to 29 taps) through a buffer that starts at the
    // dword boundary at or below w, and shifted down 2 bytes when the run
    // starts between dwords. A run whose 64 bytes would reach past w's end
    // (only the last runs of w) is read tap by tap.
    constexpr int kRunDW = 16;   // dwords loaded per run
    const uint32_t wal = (uint32_t)((uintptr_t)w & 3);
    const uint32_t wrng = a.worig + wal;
    auto gather_w_runs = [&](int g, int sb) {
        constexpr int NPR = 8 * kCoW / kNTW;
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(w, a.worig);
        const __amdgpu_buffer_rsrc_t ra =
            raw_rsrc(reinterpret_cast<const unsigned char*>(w) - wal, wrng);
        unsigned short* F = reinterpret_cast<unsigned short*>(smem + (size_t)sb * a.stage_bytes);
        uint32_t d[NPR][kRunDW];
        uint32_t src[NPR], sh[NPR];
        bool tail[NPR];
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
            const int pr = tid + p * kNTW, k = pr >> 3, c = pr & 7;
            const int co = co0 + k, ch = 8 * g + c;
            src[p] = co < Co && ch < Ci ? (uint32_t)(((int64_t)co * Ci + ch) * HW * 2) : kMissW;
            const uint32_t sa = (src[p] + wal) & ~3u;
            tail[p] = src[p] != kMissW && sa + 4 * kRunDW > wrng;
            const bool hit = src[p] != kMissW && !tail[p];
            sh[p] = ((src[p] + wal) & 2u) * 8u;
#pragma unroll
            for (int q = 0; q < kRunDW / 4; ++q) {
                const auto u = __builtin_amdgcn_raw_buffer_load_b128(
                    ra, (int)(hit ? sa + 16 * q : kMissW), 0, 0);
                d[p][4 * q] = u[0];
                d[p][4 * q + 1] = u[1];
                d[p][4 * q + 2] = u[2];
                d[p][4 * q + 3] = u[3];
            }
        }
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
            const int pr = tid + p * kNTW;
            const int dst = pr;   // (k, c): half k*8 + c of each tap's 2 KB
            if (tail[p]) {
#pragma unroll
                for (int j = 0; j < 2 * kRunDW - 2; ++j)
                    if (j < a.HWp)
                        F[j * kCoW * 8 + dst] = (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(
                            r, (int)(j < HW ? src[p] + 2 * j : kMissW), 0, 0);
                continue;
            }
#pragma unroll
            for (int j = 0; j < 2 * kRunDW - 2; ++j) {
                if (j >= a.HWp) break;
                const uint32_t dw = __builtin_amdgcn_alignbit(d[p][(j >> 1) + 1], d[p][j >> 1], sh[p]);
                const uint32_t hv = j < HW ? (dw >> (16 * (j & 1))) & 0xFFFFu : 0u;
                F[j * kCoW * 8 + dst] = (unsigned short)hv;
            }
        }
    };

    // Window offsets of the taps in filter order j = kh*Wf + kw, from the
    // pixel's tap (0, 0): kh*RS + (kw % sw)*NU + kw / sw. Entries from HW on
    // repeat tap HW-1 (reads of those are unused or zeroed).
    int* T = reinterpret_cast<int*>(smem + a.tab);
    for (int j = tid; j < a.KT; j += kNTW) {
        const int jj = j < HW ? j : HW - 1;
        const int kh = jj / Wf, kw = jj - (jj / Wf) * Wf;
        T[j] = kh * RS + (kw % sw) * NU + kw / sw;
    }

    floatx16_t acc[4][kNBW];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < kNBW; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][b][r] = 0.f;

    // Fragments of one tap pair: taps 2t (lanes 0-31) and 2t+1 (32-63); A for
    // the four 32-channel blocks, B for the four pixel blocks. on0 and on1
    // hold this lane's window offsets of the next two pairs.
    struct Frags {
        half8_t a[4], b[kNBW];
    };
    int on0 = 0, on1 = 0;
    const uint4* A = nullptr;
    const uint4* X = nullptr;
    auto fetch = [&](Frags& f, int t) {
        const int o = on0;
        on0 = on1;
        on1 = T[2 * t + 4 + hl];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 u = A[(2 * t + hl) * kCoW + i * 32 + l32];
            __builtin_memcpy(&f.a[i], &u, 16);
        }
#pragma unroll
        for (int b = 0; b < kNBW; ++b) {
            const uint4 u = X[xb[b] + o];
            __builtin_memcpy(&f.b[b], &u, 16);
        }
    };
    auto mma = [&](const Frags& f) {
#pragma unroll
        for (int b = 0; b < kNBW; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[i], f.b[b], acc[i][b], 0, 0, 0);
    };

    const int nfull = HW >> 1;          // tap pairs with two real taps
    const bool odd = (HW & 1) != 0;

    // sync: one buffer; group g's filter and rows are copied through
    // registers after every wave is done with group g-1, and its MFMAs start
    // once they have landed (no copy in flight during the MFMAs).
    const bool sync = a.sync;
    // Stage 0.
    if (WPK) {
        if (sync) copy_w(0, 0); else dma_w(0, 0);
    } else {
        if (HW <= 2 * kRunDW - 3) gather_w_runs(0, 0); else gather_w(0, 0);
    }
    load_x(0);
    store_x(0);
    __syncthreads();   // the tap table
    // Window offsets of the first two pairs, the same in every group.
    const int t0 = T[hl], t1 = T[2 + hl];
    for (int g = 0; g < a.CG; ++g) {
        if (sync && g > 0) {
            __syncthreads();   // every wave is done with group g-1
            if (WPK) copy_w(g, 0); else if (HW <= 2 * kRunDW - 3) gather_w_runs(g, 0); else gather_w(g, 0);
            load_x(g);
            store_x(0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's filter loads of group g
        __syncthreads();   // every wave's loads and input rows; buffer (g+1)%2 is free
        const size_t sb = sync ? 0 : (size_t)(g & 1);
        A = reinterpret_cast<const uint4*>(smem + sb * a.stage_bytes);
        X = reinterpret_cast<const uint4*>(smem + sb * a.stage_bytes + a.fbytes);

        // The fragments of pair t+1 are read while the MFMAs of pair t run;
        // reads run at most two pairs past the group (inside the allocation,
        // never used). The first pair's reads go out before the next group's
        // loads are issued.
        Frags f0, f1;
        on0 = t0;
        on1 = t1;
        fetch(f0, 0);
        if (!sync && g + 1 < a.CG) {
            if (WPK) dma_w(g + 1, (g + 1) & 1);
            load_x(g + 1);
        }
        int t = 0;
        for (; t + 2 <= nfull; t += 2) {
            fetch(f1, t + 1);
            __builtin_amdgcn_sched_barrier(0);
            mma(f0);
            __builtin_amdgcn_sched_barrier(0);
            fetch(f0, t + 2);
            __builtin_amdgcn_sched_barrier(0);
            mma(f1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Left: f0 = pair t.
        if (t < nfull) {
            if (odd) fetch(f1, t + 1);
            mma(f0);
            f0 = f1;
        }
        if (odd) {
            // Last tap with a zero partner: its filter entry is zero in the
            // prepacked filter and lanes 32-63 zero their B slice, so an
            // infinity next to a window cannot turn into NaN.
            const uint32_t keep = hl ? 0u : ~0u;
#pragma unroll
            for (int b = 0; b < kNBW; ++b) {
                uint4 u;
                __builtin_memcpy(&u, &f0.b[b], 16);
                u.x &= keep; u.y &= keep; u.z &= keep; u.w &= keep;
                __builtin_memcpy(&f0.b[b], &u, 16);
            }
            mma(f0);
        }
        if (!sync && g + 1 < a.CG) {
            store_x((g + 1) & 1);
            if (!WPK) {
                if (HW <= 2 * kRunDW - 3) gather_w_runs(g + 1, (g + 1) & 1); else gather_w(g + 1, (g + 1) & 1);
            }
        }
    }

    // Output: lane holds pixel l32 of each block and channels
    // 8*(r/4) + 4*hl + r%4 of each 32-channel block. Blocks 2p and 2p+1 of a
    // wave are 64 consecutive pixels: swapping lanes 32-63 of the first with
    // lanes 0-31 of the second (v_permlane32_swap) gives one register with
    // channel cu for all 64 pixels and one with channel cu+4, so every store
    // writes 256 contiguous bytes of one channel plane (32-pixel stores into
    // two planes made the HBM writes about 1.3x the output).
    const int64_t plane = (int64_t)Ho * Wo;
    const __amdgpu_buffer_rsrc_t yb = raw_rsrc(y, a.ybytes);
    const bool all_co = co0 + kCoW <= Co;
#pragma unroll
    for (int p = 0; p < kNBW / 2; ++p) {
        const int64_t qa = q0 + (wave * kNBW + 2 * p) * 32 + lane;
        const bool ok = qa < qend;
        const int64_t q = ok ? qa : qend - 1;
        const int gr = (int)(q / Wo);
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int n = (int)a.divHo.div((uint32_t)gr), ho = gr - n * Ho;
        const uint32_t vo = (uint32_t)((((int64_t)n * Co) * plane + (int64_t)ho * Wo + wo) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
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

// Plans a launch; false if the shape is outside the kernel's envelope:
// Co >= 128 (a tile's 128 channels are mostly real), the stage fits LDS
// twice over, the input rows fit the per-thread staging capacity, tensors
// addressable with 32-bit buffer offsets. Knobs (tuning and tests):
// KNOB_F16_WIDE < 0 turns the kernel off, > 0 lets it take Co < 128 too.
bool plan(const ConvShape& c, WideArgs& a, size_t copad_mult)
{
    const int sw_knob = knob(KNOB_F16_WIDE);
    if (sw_knob < 0) return false;
    if (c.Co < kCoW && sw_knob <= 0) return false;
    a.c = c;
    a.HW = c.Hf * c.Wf;
    a.HWp = (a.HW + 1) & ~1;
    a.CG = ceil_div(c.Ci, 8);
    a.KT = (a.HWp + 8 + 3) & ~3;
    a.Copad = (int)(ceil_div(c.Co, (int)copad_mult) * (int)copad_mult);
    a.total = (int64_t)c.N * c.Ho * c.Wo;
    a.dup = std::max(0, c.Hf - c.sh);
    if ((int64_t)c.N * c.Ho > 0x7fffffff) return false;
    const int64_t plane = (int64_t)c.Ho * c.Wo;
    a.rows_max = (int)std::min<int64_t>((kPW - 1) / c.Wo + 2, (int64_t)c.N * c.Ho);
    a.tiles_per_image = (plane + kPW - 1) / kPW;
    a.aligned = (double)(a.tiles_per_image * kPW) <= 1.05 * (double)plane;
    a.kmax = a.aligned || a.rows_max <= 1 ? 0 : std::min(c.N - 1, ceil_div(a.rows_max - 1, c.Ho));
    a.RIN = (a.rows_max - 1) * c.sh + c.Hf + a.kmax * a.dup;
    a.NU = ceil_div(c.Wi, c.sw);
    a.RS = c.sw * a.NU;
    a.xentries = a.RIN * a.RS;
    const bool xpair = c.Wi % 2 == 0;
    a.xunits = xpair ? a.RIN * (c.Wi / 2) : a.RIN * c.Wi;
    if (a.xunits > (xpair ? kXUW : kXEW)) return false;
    a.S = 2 * a.HWp;
    a.fbytes = (uint32_t)a.HWp * kCoW * 16;
    a.stage_bytes = a.fbytes + (uint32_t)a.xentries * 16;
    a.tab = 2 * a.stage_bytes;
    a.lds_bytes = a.tab + (uint32_t)((a.KT * 4 + 15) / 16 * 16) + kSlackW;
    if (a.lds_bytes > (uint32_t)kWideLds) return false;
    a.co_tiles = ceil_div(c.Co, kCoW);
    a.px_tiles = a.aligned ? (int64_t)c.N * a.tiles_per_image : (a.total + kPW - 1) / kPW;
    if (a.px_tiles * a.co_tiles > 0x7fffffff) return false;
    const int64_t xb = (int64_t)c.N * c.Ci * c.Hi * c.Wi * 2;
    const int64_t yb = (int64_t)c.N * c.Co * c.Ho * c.Wo * 4;
    const int64_t wb = (int64_t)a.CG * a.HWp * a.Copad * 16;
    const int64_t wo = (int64_t)c.Co * c.Ci * a.HW * 2;
    if (xb >= (int64_t)kMissW || yb >= (int64_t)kMissW || wb >= (int64_t)kMissW ||
        wo >= (int64_t)kMissW)
        return false;
    a.worig = (uint32_t)wo;
    a.xbytes = (uint32_t)xb;
    a.ybytes = (uint32_t)yb;
    a.wbytes = (uint32_t)wb;
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divHo = FastDiv((uint32_t)c.Ho);
    a.divWi = FastDiv((uint32_t)c.Wi);
    a.divHalfW = FastDiv((uint32_t)std::max(1, c.Wi / 2));
    a.divS = FastDiv((uint32_t)c.sw);
    a.swz = knob(KNOB_TILE_ORDER) != 1;
    a.sync = knob(KNOB_SYNC_STAGING) == 1;
    return true;
}

template <int NW, int NB, bool XPAIR, bool WPK>
int launch_t(const uint16_t* x, const uint4* wpk, const uint16_t* w, float* y, const WideArgs& a,
             hipStream_t stream)
{
    ensure_lds_limit((const void*)conv_f16_wide_kernel<NW, NB, XPAIR, WPK>, kWideLds);
    hipLaunchKernelGGL((conv_f16_wide_kernel<NW, NB, XPAIR, WPK>),
                       dim3((unsigned)(a.px_tiles * a.co_tiles)), dim3(64 * NW), a.lds_bytes,
                       stream, x, wpk, w, y, a);
    return launch_status();
}

template <int NW, int NB, bool WPK>
int launch_x(const uint16_t* x, const uint4* wpk, const uint16_t* w, float* y, const WideArgs& a,
             hipStream_t stream)
{
    return a.c.Wi % 2 == 0 ? launch_t<NW, NB, true, WPK>(x, wpk, w, y, a, stream)
                           : launch_t<NW, NB, false, WPK>(x, wpk, w, y, a, stream);
}

}  // namespace

bool f16_wide_applies(const ConvShape& c, size_t copad_mult)
{
    WideArgs a;
    return plan(c, a, copad_mult);
}

int launch_conv_f16_wide(const uint16_t* x, const void* wpk, const uint16_t* w, float* y,
                         const ConvShape& c, size_t copad_mult, hipStream_t stream)
{
    WideArgs a;
    if (copad_mult % kCoW != 0) return -1;
    if (!plan(c, a, copad_mult)) return -1;
    if ((uintptr_t)wpk % 16 != 0) return -1;
    const uint4* w4 = static_cast<const uint4*>(wpk);
    // KNOB_F16_WIDE_NW: 4 waves of 4 x 4 blocks, or (default) 8 waves of 4 x 2.
    const bool nw4 = knob(KNOB_F16_WIDE_NW) == 4;
    if (w4) return nw4 ? launch_x<4, 4, true>(x, w4, w, y, a, stream)
                       : launch_x<8, 2, true>(x, w4, w, y, a, stream);
    return nw4 ? launch_x<4, 4, false>(x, w4, w, y, a, stream)
               : launch_x<8, 2, false>(x, w4, w, y, a, stream);
}

}  // namespace im2win
