// fp32 im2win convolution on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The single-precision path of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract: full
// precision; Fig. 1: the convolution as dot products of filters with im2win
// windows) for one MI355X. fp32 products and fp32 accumulation, as on the
// vector ALUs, but at the matrix-core rate (twice the unpacked vector FMA
// rate):
//
//  * GEMM view: rows = output channels (A = filters), columns = output
//    pixels (B = windows), K = (input channel, kh, kw) in the filter's own
//    memory order. Pixels are numbered over the whole batch,
//    q = (n*Ho + ho)*Wo + wo. A workgroup of NW waves owns 32*WCO channels
//    and 32*NW/KSW consecutive pixels; wave v owns the 32-pixel block
//    v % (NW/KSW) of the tile and all 32*WCO channels (WCO MFMA tiles,
//    AGPR accumulators).
//  * A stage is CB input channels. Per stage the workgroup stages in LDS the
//    input rows its pixels' windows cover (one fp32 per entry, columns
//    stride-phase major so the 32 pixels of a block read 32 consecutive
//    entries for every tap) and the filter rows w[co][ci0..ci0+CB)[*] as
//    they lie in memory, one LDS row per channel at an odd pitch, so the 32
//    lanes reading one K index hit 32 different banks.
//  * One MFMA consumes two consecutive K indices (lanes 0-31 the even one,
//    32-63 the odd one); an odd K count per stage gets a zero filter entry
//    and a zeroed window value, so an infinity next to a window never turns
//    into NaN.
//  * The next stage's global loads are issued into registers before the
//    MFMAs of the current stage and written to LDS after them.
//  * Small problems (too few tiles to fill the chip) split K inside the
//    workgroup: KSW waves share each pixel block, each taking a contiguous
//    range of every stage's K pairs, and their partial sums are added
//    through LDS in a fixed order (wave share 0 + 1 + ... + KSW-1) before
//    the store, so results do not depend on timing.
#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"
#include "knobs.hpp"

namespace im2win {

namespace {

constexpr int kMaxLds = 160 * 1024;
// Input rows per wave and stage for NW waves (32, 40 or 48 per workgroup).
constexpr int rows_per_wave(int nw) { return nw == 4 ? 8 : nw == 8 ? 5 : 4; }
constexpr uint32_t kMaxBuf = 0xFFFFFFF0u;   // buffer ranges are 32-bit

struct MArgs {
    ConvShape c;
    int co_tiles;                     // channel tiles
    int64_t px_tiles, total, tiles_per_image;
    bool aligned;                     // tiles never cross images
    int rows_max, kmax, dup, RIN;     // output rows per tile, image breaks, sh<Hf overlap, LDS rows
    int HW, CB, nstages, KSP, KT;     // taps; channels per stage; stages; filter row pitch (odd);
                                      // K offset table entries
    int NU, RS, CSX, xent;            // entries per phase, per row (sw*NU), per channel; total
    uint32_t xbytes, wbytes, ybytes;
    bool swz;                         // XCD-grouped item order
    bool sync;                        // next stage loaded after this one's MFMAs
    FastDiv divWo, divHo, divS;
};

// Buffer resources (raw_rsrc) cover [base, base + bytes): loads at soffset +
// voffset + offset >= bytes return 0 (the scalar offset counts in the range
// check).
// The staging loads below use one resource per tensor, so a load past the
// end of a row reads the next row (or 0 past the tensor) and is not stored.

template <int NW, int KSW, int WCO, int XCH, int WCH>
__global__ __launch_bounds__(64 * NW) void conv_f32_mfma_kernel(
    const float* __restrict__ x, const float* __restrict__ w, float* __restrict__ y, MArgs a)
{
    constexpr int NT = 64 * NW;
    constexpr int NPB = NW / KSW;                 // 32-pixel blocks per tile
    constexpr int P = 32 * NPB;                   // pixels per tile
    constexpr int COT = 32 * WCO;
    constexpr int RPW = rows_per_wave(NW);        // input rows per wave and stage
    constexpr int WRW = (COT + NW - 1) / NW;      // filter rows per wave and stage
    constexpr int KSP = 64 * WCH + 1;             // filter row pitch in LDS (odd)

    extern __shared__ __align__(16) float lds[];
    float* X = lds;
    float* Wl = lds + a.xent;
    int* T = reinterpret_cast<int*>(Wl + WRW * NW * KSP);   // after WRW*NW filter rows

    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co;
    const int sh = a.c.sh, sw = a.c.sw;
    const int Ho = a.c.Ho, Wo = a.c.Wo, Hf = a.c.Hf, Wf = a.c.Wf;
    const int HW = a.HW, RS = a.RS, NU = a.NU, RIN = a.RIN, CB = a.CB;
    const int64_t plane = (int64_t)Ho * Wo;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int wave = uniform(tid >> 6);
    const int pbk = wave % NPB;    // this wave's pixel block
    const int kgr = wave / NPB;    // this wave's share of each stage's K pairs

    // Work items (channel tile, pixel tile), item = pixel tile * co_tiles +
    // channel tile. A workgroup takes items blockIdx.x, blockIdx.x +
    // gridDim.x, ... and streams their stages back to back, so the next
    // item's first stage is fetched while the current item's last stage runs.
    const int64_t items = a.px_tiles * a.co_tiles;
    struct Item {
        int co0, st0, st1, gr0, grl, n0;
        int64_t q0, qend;
    };
    auto item_of = [&](int64_t it, Item& m) {
        const int co_t = (int)(it % a.co_tiles);
        const int64_t pt = it / a.co_tiles;
        m.co0 = co_t * COT;
        m.st0 = 0;
        m.st1 = a.nstages;
        if (a.aligned) {   // pixel tile = (image, tile within the image)
            const int64_t img = pt / a.tiles_per_image;
            m.q0 = img * plane + (pt - img * a.tiles_per_image) * P;
            m.qend = min(m.q0 + P, (img + 1) * plane);
        } else {
            m.q0 = pt * P;
            m.qend = m.q0 + P < a.total ? m.q0 + P : a.total;
        }
        m.gr0 = (int)(m.q0 / Wo);
        m.grl = (int)((m.qend - 1) / Wo);
        m.n0 = (int)a.divHo.div((uint32_t)m.gr0);
    };

    // LDS row i of item m -> (image n, input row h); false if no input row
    // maps there. Segment k holds the output rows of image n0+k in the tile,
    // at LDS rows (first - gr0)*sh + k*dup onwards.
    auto x_src = [&](const Item& m, int i, int& n, int& h) -> bool {
        for (int k = 0; k <= a.kmax; ++k) {
            const int nk = m.n0 + k;
            const int first = max(m.gr0, nk * Ho), last = min(m.grl, nk * Ho + Ho - 1);
            if (first > last) break;
            const int S = (first - m.gr0) * sh + k * a.dup;
            const int span = (last - first) * sh + Hf;
            if (i >= S && i < S + span) {
                n = nk;
                h = (first - nk * Ho) * sh + (i - S);
                return true;
            }
        }
        return false;
    };

    // Offsets of the K indices of a stage (channel cl, kh, kw in filter
    // order) from a pixel's tap (0, 0) of channel 0: cl*CSX + kh*RS +
    // (kw % sw)*NU + kw / sw. Tabulated once per workgroup so that each lane
    // reads its own index's offset (one LDS read per pair) instead of walking
    // the taps on the scalar unit. Entries past the stage read as offset 0.
    for (int k = tid; k < a.KT; k += NT) {
        int off = 0;
        if (k < CB * HW) {
            const int cl = k / HW, j = k - (k / HW) * HW;
            const int kh = j / Wf, kw = j - (j / Wf) * Wf;
            off = cl * a.CSX + kh * RS + (kw % sw) * NU + kw / sw;
        }
        T[k] = off;
    }

    // ---- staging (load side: item L) ---------------------------------------
    // Wave v stages LDS rows r = v + NW*ii of a stage (channel r / RIN, row
    // r % RIN), its lanes taking columns lane + 64*cc: the row's byte offset
    // in x is the scalar offset of the load, the column the vector offset.
    // Filter rows co = v + NW*i, lanes taking taps lane + 64*jc. There are no
    // per-row or per-lane branches: a row with no source gets a scalar offset
    // past the end of x (it loads zeros) and is written to a spare LDS row;
    // every lane column has an entry in its row (rows are padded to 64*XCH
    // columns; those past Wi are never read); every lane tap has an entry in
    // its filter row (pitch 64*WCH + 1).
    Item L;
    uint32_t xrow[RPW];   // byte offset in x from the stage's first channel, or past the end
    int xdr[RPW];         // LDS row written (the spare row CB*RIN if none)
    auto setup_load = [&](const Item& m) {
#pragma unroll
        for (int ii = 0; ii < RPW; ++ii) {
            const int r = wave + NW * ii;
            const int cl = r / RIN, i = r - (r / RIN) * RIN;
            int n = 0, h = 0;
            const bool ok = cl < CB && x_src(m, i, n, h);
            xrow[ii] = ok ? (uint32_t)(((((int64_t)n * Ci + cl) * Hi + h) * Wi) * 4) : a.xbytes;
            xdr[ii] = ok ? r : CB * RIN;
        }
    };
    const uint32_t lane4 = (uint32_t)lane * 4;
    int xdst[XCH];   // LDS entry of column lane + 64*cc within a row
#pragma unroll
    for (int cc = 0; cc < XCH; ++cc) {
        const int col = lane + 64 * cc;
        const int u = (int)a.divS.div((uint32_t)col);
        xdst[cc] = (col - u * sw) * NU + u;
    }
    float xv[RPW][XCH];
    float wv[WRW][WCH];
    const uint32_t wpitch = (uint32_t)Ci * HW * 4;   // bytes between filters
    const __amdgpu_buffer_rsrc_t xr = raw_rsrc(x, a.xbytes);

    auto load_stage = [&](int st) {
        const int ci0 = st * CB;
        // Opaque per stage, so the per-row offsets below are recomputed here
        // rather than kept live across the stage loop.
        uint32_t cofs = (uint32_t)ci0 * Hi * Wi * 4;
        asm volatile("" : "+s"(cofs));
#pragma unroll
        for (int ii = 0; ii < RPW; ++ii) {
            const uint32_t so = xrow[ii] + cofs;
#pragma unroll
            for (int cc = 0; cc < XCH; ++cc)
                xv[ii][cc] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    xr, (int)(lane4 + 256 * cc), (int)so, 0));
        }
        // Filters co0 + co, channels ci0 .. ci0 + cbs - 1: cbs*HW contiguous
        // taps each (what a lane reads past them is replaced by zero when
        // stored). Filters past Co read zeros (offset past the end).
        const int64_t wfirst = ((int64_t)L.co0 * Ci + ci0) * HW;
        const uint32_t wrange = a.wbytes - (uint32_t)(wfirst * 4);
        const __amdgpu_buffer_rsrc_t wr = raw_rsrc(w + wfirst, wrange);
        int nco = Co - L.co0;   // filters left from co0
        asm volatile("" : "+s"(nco));
#pragma unroll
        for (int i = 0; i < WRW; ++i) {
            const int co = wave + NW * i;
            const uint32_t so = co < nco ? (uint32_t)co * wpitch : wrange;
#pragma unroll
            for (int jc = 0; jc < WCH; ++jc)
                wv[i][jc] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    wr, (int)(lane4 + 256 * jc), (int)so, 0));
        }
    };
    auto store_stage = [&](int st) {
        const int ks = min(CB, Ci - st * CB) * HW;
        int rsb = RS * 4;   // opaque per stage (see load_stage)
        asm volatile("" : "+s"(rsb));
#pragma unroll
        for (int ii = 0; ii < RPW; ++ii) {
            char* row = reinterpret_cast<char*>(X) + xdr[ii] * rsb;
#pragma unroll
            for (int cc = 0; cc < XCH; ++cc)
                *reinterpret_cast<float*>(row + xdst[cc] * 4) = xv[ii][cc];
        }
#pragma unroll
        for (int i = 0; i < WRW; ++i) {
            float* row = Wl + (wave + NW * i) * KSP;
#pragma unroll
            for (int jc = 0; jc < WCH; ++jc) {
                const int j = lane + 64 * jc;
                row[j] = j < ks ? wv[i][jc] : 0.f;
            }
        }
    };

    // ---- compute side (item C) ----------------------------------------------
    // This lane's pixel: entry of its tap (0, 0) in a channel's LDS rows
    // (output row gr: tile-relative r*sh plus image breaks k*dup), and where
    // its outputs go.
    Item C;
    int xb = 0;
    auto setup_compute = [&]() {
        int64_t q = C.q0 + pbk * 32 + l32;
        if (q >= C.qend) q = C.qend - 1;
        const int gr = (int)a.divWo.div((uint32_t)(q - (int64_t)C.gr0 * Wo)) + C.gr0;
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int k = (int)a.divHo.div((uint32_t)gr) - C.n0;
        xb = ((gr - C.gr0) * sh + k * a.dup) * RS + wo;
    };
    const int abase = l32 * KSP + hl;   // A: channel l32 of each block, K index 2t + hl

    floatx16_t acc[WCO];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < WCO; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    };

    struct Frags {
        float a[WCO], b;
    };
    // Fragments of pair t: this lane's K index is 2t + hl. The window offsets
    // of pairs t and t+1 are held in on0, on1 (read from T two pairs ahead),
    // so a window read never waits on a table read issued just before it.
    int on0 = 0, on1 = 0;
    auto fetch = [&](Frags& f, int t) {
        const int o = on0;
        on0 = on1;
        on1 = T[2 * t + 4 + hl];
        f.b = X[xb + o];
#pragma unroll
        for (int i = 0; i < WCO; ++i) f.a[i] = Wl[abase + i * 32 * KSP + 2 * t];
    };
    auto mma = [&](const Frags& f) {
#pragma unroll
        for (int i = 0; i < WCO; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i], f.b, acc[i], 0, 0, 0);
    };
    auto compute_stage = [&](int st) {
        const int ks = min(CB, Ci - st * CB) * HW;
        // This wave's pairs [t0, t1) of the stage's (ks + 1) / 2; with ks
        // odd the stage's last pair is half empty (odd_last: this wave has
        // it) and nfull ends the pairs with two real K indices.
        const int np = (ks + 1) >> 1;
        int t0 = 0, t1 = np;
        if (KSW > 1) {
            const int per = (np + KSW - 1) / KSW;
            t0 = min(np, kgr * per);
            t1 = min(np, t0 + per);
        }
        const bool odd_last = (ks & 1) && t1 == np && t0 < t1;
        const int nfull = odd_last ? t1 - 1 : t1;
        if (t0 >= t1) return;
        // Pair t+1 is read from LDS while the MFMAs of pair t run. The loop
        // body fetches unconditionally (one pair past the end at most: an
        // in-allocation read that is never used), so every path into an
        // MFMA has the same reads outstanding and the waits stay exact.
        Frags f0, f1;
        on0 = T[2 * t0 + hl];
        on1 = T[2 * t0 + 2 + hl];
        fetch(f0, t0);
        int t = t0;
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
        // Left: f0 = pair t. Pair nfull, if odd_last, is the last K index
        // with a zero partner: filter entry ks is zero and lanes 32-63 zero
        // their window value.
        if (t < nfull) {
            mma(f0);
            if (odd_last) fetch(f0, nfull);
            ++t;
        }
        if (odd_last) {
            f0.b = hl ? 0.f : f0.b;
            mma(f0);
        }
    };

    // Partial sums of the K shares (KSW > 1): shares 1 .. KSW-1 leave theirs
    // in LDS past the offset table (one 4 KB block per share, pixel block
    // and channel block: register r of lane l at float r*64 + l), and share
    // 0 adds them in share order before the store. Every wave takes part in
    // the barrier; the loop's next barrier keeps the area from being
    // rewritten before share 0 has read it.
    auto reduce_shares = [&]() {
        float* R = reinterpret_cast<float*>(T + a.KT);
        if (kgr > 0) {
            float* d = R + (((kgr - 1) * NPB + pbk) * WCO) * 1024 + lane;
#pragma unroll
            for (int i = 0; i < WCO; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) d[(i * 16 + r) * 64] = acc[i][r];
        }
        __syncthreads();
        if (kgr == 0) {
            for (int g = 1; g < KSW; ++g) {
                const float* s = R + (((g - 1) * NPB + pbk) * WCO) * 1024 + lane;
#pragma unroll
                for (int i = 0; i < WCO; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][r] += s[(i * 16 + r) * 64];
            }
        }
    };

    // Output of item C: lane holds pixel l32 of its block and channels
    // 8*(r/4) + 4*hl + r%4 of each 32-channel block.
    auto epilogue = [&]() {
        if (KSW > 1) {
            reduce_shares();
            if (kgr > 0) return;
        }
        const int64_t qme = C.q0 + pbk * 32 + l32;
        const bool qok = qme < C.qend;
        const int64_t q = qok ? qme : C.qend - 1;
        const int gr = (int)(q / Wo);
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int n = (int)a.divHo.div((uint32_t)gr), ho = gr - n * Ho;
        const int co0 = C.co0;
        const bool all_co = co0 + COT <= Co;
        // Byte offset = per-lane part (image, pixel, 4*hl channels) +
        // uniform part (channel block row).
        const __amdgpu_buffer_rsrc_t yb = raw_rsrc(y, a.ybytes);
        const uint32_t voff =
            (uint32_t)((((int64_t)n * Co + 4 * hl) * plane + (int64_t)ho * Wo + wo) * 4);
        if (qok) {
#pragma unroll
            for (int i = 0; i < WCO; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int cu = co0 + i * 32 + 8 * (r >> 2) + (r & 3);   // channel - 4*hl
                    const float v = acc[i][r];
                    if (all_co || cu + 4 * hl < Co)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), yb, (int)voff,
                                                              (int)(cu * plane * 4), 0);
                }
        }
    };

    // ---- the step stream ------------------------------------------------------
    // Workgroups of one XCD take neighbouring items (XCD-grouped order)
    // unless the tile_order knob asks for launch order; either way the
    // first items are a permutation of 0 .. gridDim.x - 1.
    int64_t it = xcd_tile(blockIdx.x, gridDim.x, a.swz);
    if (it >= items) return;
    item_of(it, L);
    setup_load(L);
    load_stage(L.st0);
    store_stage(L.st0);
    __syncthreads();
    C = L;
    setup_compute();
    zero_acc();
    int st = C.st0;
    for (;;) {
        // Next step: the next stage of this item, or the first of the next.
        const bool last = st + 1 == C.st1;
        int nst = st + 1;
        int64_t nit = it;
        bool more = true;
        if (last) {
            nit = it + gridDim.x;
            more = nit < items;
            if (more) {
                item_of(nit, L);
                setup_load(L);
                nst = L.st0;
            }
        }
        // sync: the next stage's loads wait until this stage's MFMAs are
        // issued, so no copy is in flight while they run.
        if (more && !a.sync) load_stage(nst);
        compute_stage(st);
        if (last) {
            epilogue();
            zero_acc();
        }
        if (!more) break;
        __syncthreads();
        if (a.sync) load_stage(nst);
        store_stage(nst);
        __syncthreads();
        if (last) {
            it = nit;
            C = L;
            setup_compute();
        }
        st = nst;
    }
}

// Geometry of a launch with NW waves, KSW of them sharing each pixel block
// (32*NW/KSW pixels per tile), and 32*WCO channels per tile; false if the
// shape is outside the kernel's envelope.
bool plan(const ConvShape& c, int nw, int ksw, int wco, MArgs& a, int& xch, int& wch)
{
    a.c = c;
    a.HW = c.Hf * c.Wf;
    a.total = (int64_t)c.N * c.Ho * c.Wo;
    a.dup = std::max(0, c.Hf - c.sh);
    if ((int64_t)c.N * c.Ho > 0x7fffffff) return false;
    xch = ceil_div(c.Wi, 64);
    if (xch == 3) xch = 4;
    if (xch > 4 || a.HW > 254) return false;
    const int P = 32 * (nw / ksw), cot = 32 * wco, rows_cap = nw * rows_per_wave(nw);
    const int64_t red = (int64_t)(ksw - 1) * (nw / ksw) * wco * 4096;   // K-share partial sums
    const int wrows = (cot + nw - 1) / nw * nw;   // filter rows staged (>= cot)

    // Entries per stride phase: every lane column (64*xch of them) has one.
    a.NU = ceil_div(64 * xch, c.sw);
    a.RS = c.sw * a.NU;
    const int64_t plane = (int64_t)c.Ho * c.Wo;
    a.rows_max = (P - 1) / c.Wo + 2;
    a.tiles_per_image = (plane + P - 1) / P;
    a.aligned = c.N == 1 || (double)(a.tiles_per_image * P) <= 1.05 * (double)plane;
    a.kmax = a.aligned || a.rows_max <= 1 ? 0 : ceil_div(a.rows_max - 1, c.Ho);
    a.RIN = (a.rows_max - 1) * c.sh + c.Hf + a.kmax * a.dup;
    if (a.RIN > rows_cap) return false;
    a.CSX = a.RIN * a.RS;

    // Channels per stage: fill the row slots, keep the filter rows within
    // the register prefetch (instantiated chunk counts) and the LDS budget.
    auto wch_of = [&](int cb) {
        const int v = ceil_div(cb * a.HW + 1, 64);   // taps plus the odd-K pad entry
        return v == 3 ? 4 : v;
    };
    auto wregs = [&](int cb) { return wrows / nw * wch_of(cb); };
    auto lds_of = [&](int cb) {
        return (((int64_t)cb * a.RIN + 1) * a.RS + (int64_t)wrows * (64 * wch_of(cb) + 1) +
                cb * a.HW + 12) * 4 + red;
    };
    auto fits = [&](int cb, int64_t budget) {
        return wch_of(cb) <= 2 && wregs(cb) <= 48 && lds_of(cb) <= budget;
    };
    int cb = std::min(c.Ci, rows_cap / a.RIN);
    while (cb > 1 && !fits(cb, 80 * 1024)) --cb;
    if (knob(KNOB_F32_CB) > 0) cb = std::min(cb, knob(KNOB_F32_CB));
    if (!fits(cb, kMaxLds)) return false;
    wch = wch_of(cb);
    a.CB = cb;
    a.KSP = 64 * wch + 1;
    a.xent = (cb * a.RIN + 1) * a.RS;   // plus one spare row
    a.KT = (cb * a.HW + 8 + 3) & ~3;    // reads reach index ks + 7
    a.nstages = ceil_div(c.Ci, cb);
    a.co_tiles = ceil_div(c.Co, cot);
    a.px_tiles = a.aligned ? (int64_t)c.N * a.tiles_per_image : (a.total + P - 1) / P;
    if (a.px_tiles * a.co_tiles > 0x7fffffff) return false;

    // Scalar offsets and buffer ranges are 32-bit; a row with no source uses
    // an offset of xbytes plus a channel offset below xbytes.
    const int64_t xb = (int64_t)c.N * c.Ci * c.Hi * c.Wi * 4;
    const int64_t yb = (int64_t)c.N * c.Co * c.Ho * c.Wo * 4;
    const int64_t wb = (int64_t)c.Co * c.Ci * a.HW * 4;
    if (2 * xb >= (int64_t)kMaxBuf || yb >= (int64_t)kMaxBuf || wb >= (int64_t)kMaxBuf)
        return false;
    a.xbytes = (uint32_t)xb;
    a.wbytes = (uint32_t)wb;
    a.ybytes = (uint32_t)yb;
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divHo = FastDiv((uint32_t)c.Ho);
    a.divS = FastDiv((uint32_t)c.sw);
    return true;
}

size_t lds_bytes(const MArgs& a, int nw, int ksw, int wco)
{
    const int wrows = (32 * wco + nw - 1) / nw * nw;
    return ((size_t)a.xent + (size_t)wrows * a.KSP + a.KT) * 4 +
           (size_t)(ksw - 1) * (nw / ksw) * wco * 4096;
}

template <int NW, int KSW, int WCO, int XCH>
const void* kernel_w(int wch)
{
    if (wch == 1) return (const void*)conv_f32_mfma_kernel<NW, KSW, WCO, XCH, 1>;
    if (wch == 2) return (const void*)conv_f32_mfma_kernel<NW, KSW, WCO, XCH, 2>;
    return nullptr;
}

template <int NW, int KSW, int WCO>
const void* kernel_x(int xch, int wch)
{
    switch (xch) {
    case 1: return kernel_w<NW, KSW, WCO, 1>(wch);
    case 2: return kernel_w<NW, KSW, WCO, 2>(wch);
    case 4: return kernel_w<NW, KSW, WCO, 4>(wch);
    }
    return nullptr;
}

template <int NW>
const void* kernel_c(int wco, int xch, int wch)
{
    switch (wco) {
    case 1: return kernel_x<NW, 1, 1>(xch, wch);
    case 2: return kernel_x<NW, 1, 2>(xch, wch);
    case 3: return kernel_x<NW, 1, 3>(xch, wch);
    case 4: return kernel_x<NW, 1, 4>(xch, wch);
    }
    return nullptr;
}

// Kernels: K shares ksw of 1 (any channel tile) or NW (one pixel block and
// one 32-channel block per tile).
const void* kernel_of(int nw, int ksw, int wco, int xch, int wch)
{
    if (ksw == 1) {
        switch (nw) {
        case 4: return kernel_c<4>(wco, xch, wch);
        case 8: return kernel_c<8>(wco, xch, wch);
        case 12: return kernel_c<12>(wco, xch, wch);
        }
        return nullptr;
    }
    if (wco != 1 || ksw != nw) return nullptr;
    switch (nw) {
    case 4: return kernel_x<4, 4, 1>(xch, wch);
    case 8: return kernel_x<8, 8, 1>(xch, wch);
    case 12: return kernel_x<12, 12, 1>(xch, wch);
    }
    return nullptr;
}

std::mutex g_mu;

// Workgroups of kernel f that fit on one CU (registers and LDS), with the
// LDS limit raised to the CU's full 160 KB once per kernel. Results are
// cached per (kernel, LDS bytes, device) under a lock.
int blocks_per_cu(const void* f, int nt, size_t lds)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();   // handled: no device, the kernel is not used
        return 0;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    static std::map<std::pair<const void*, int>, bool> raised;
    static std::map<std::pair<std::pair<const void*, size_t>, int>, int> cache;
    const auto key = std::make_pair(std::make_pair(f, lds), dev);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    if (!raised.count(std::make_pair(f, dev))) {
        if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds) !=
            hipSuccess) {
            (void)hipGetLastError();   // handled: this kernel is not used
            return 0;
        }
        raised[std::make_pair(f, dev)] = true;
    }
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, nt, lds) != hipSuccess) {
        (void)hipGetLastError();   // handled: this kernel is not used
        nb = 0;
    }
    cache[key] = nb;
    return nb;
}

int cu_count()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();   // handled: assume a full MI355X
        return 256;
    }
    return n < 1 ? 256 : n;
}

struct Choice {
    MArgs a;
    int nw, ksw, wco, xch, wch;
    const void* f;
    size_t lds;
    int occ;          // workgroups that fit on a CU
    int64_t grid = 0; // persistent workgroups
    double cost;
    int wps;          // waves per SIMD
};

// Persistent grid for the work items: G = CUs*o workgroups (o <= occ), each
// taking ceil(items/G) items in turn. A wave's work per item is 32 pixels x
// the channel tile (32*WCO) x K / KSW, and a SIMD's matrix core is shared by
// its waves, so the time is ~ items per workgroup x waves per SIMD x WCO /
// KSW; ties go to more waves per SIMD (more latency hiding).
void size_grid(Choice& t, int ncu)
{
    const int64_t items = t.a.px_tiles * t.a.co_tiles;
    const int force = knob(KNOB_F32_OCC);
    t.cost = 1e300;
    t.wps = 0;
    for (int o = 1; o <= t.occ; ++o) {
        if (force > 0 && o != force) continue;
        const int64_t G = std::min<int64_t>(items, (int64_t)ncu * o);
        const int64_t per = (items + G - 1) / G;
        const int wps = (t.nw * o + 3) / 4;
        const double c = (double)per * wps * t.wco / t.ksw;
        if (c < t.cost * (1 - 1e-9) || (c < t.cost * (1 + 1e-9) && wps > t.wps)) {
            t.cost = c;
            t.wps = wps;
            t.grid = (items + per - 1) / per;
        }
    }
}

// Picks waves per workgroup, K shares, channel tile and grid.
bool choose(const ConvShape& c, Choice& ch)
{
    const int ncu = cu_count();
    int wco0 = 1, best_waste = 1 << 30;
    for (int cand = 4; cand >= 1; --cand) {
        const int waste = ceil_div(c.Co, 32 * cand) * 32 * cand - c.Co;
        if (waste < best_waste) {
            best_waste = waste;
            wco0 = cand;
        }
    }
    const int k_wco = knob(KNOB_F32_WCO), k_nw = knob(KNOB_F32_NW), k_ks = knob(KNOB_F32_KSPLIT);
    if (k_wco >= 1 && k_wco <= 4) wco0 = k_wco;

    auto make = [&](int nw, int ksw, int wc, Choice& t) -> bool {
        t.nw = nw;
        t.ksw = ksw;
        t.wco = wc;
        if (!plan(c, nw, ksw, wc, t.a, t.xch, t.wch)) return false;
        t.f = kernel_of(nw, ksw, wc, t.xch, t.wch);
        if (!t.f) return false;
        t.lds = lds_bytes(t.a, nw, ksw, wc);
        t.occ = blocks_per_cu(t.f, 64 * nw, t.lds);
        if (t.occ < 1) return false;
        size_grid(t, ncu);
        return t.wps > 0;   // false if a forced occupancy does not fit
    };
    auto better = [&](const Choice& t) {
        return t.cost < ch.cost * (1 - 1e-9) || (t.cost < ch.cost * (1 + 1e-9) && t.wps > ch.wps);
    };

    bool found = false;
    for (int wco = wco0; wco >= 1 && !found; --wco) {
        for (int nw : {12, 8, 4}) {
            if (k_nw && nw != k_nw) continue;
            Choice t;
            if (k_ks > 1 || !make(nw, 1, wco, t)) continue;
            if (!found || better(t)) {
                ch = t;
                found = true;
            }
        }
        if (k_wco) break;
    }
    // Too few tiles to fill the chip: one 32-channel block and one pixel
    // block per tile, K shared by the workgroup's waves.
    const bool small = !found || ch.a.px_tiles * ch.a.co_tiles < ncu;
    if ((small && k_ks != 1 && !k_wco) || k_ks > 1) {
        for (int nw : {12, 8, 4}) {
            if (k_nw && nw != k_nw) continue;
            if (k_ks > 1 && nw != k_ks) continue;
            Choice t;
            if (!make(nw, nw, 1, t)) continue;
            if (!found || k_ks > 1 || better(t)) {
                ch = t;
                found = true;
                if (k_ks > 1) break;
            }
        }
    }
    return found;
}

// A problem too small to fill the chip (the planner splits K inside the
// workgroup) runs on the one-stage small-problem kernel when that kernel
// takes the shape, unless a K split is forced.
bool use_small(const ConvShape& c, const Choice& ch)
{
    return ch.ksw > 1 && knob(KNOB_F32_KSPLIT) <= 0 && f32_small_applies(c);
}

}  // namespace

bool f32_mfma_applies(const ConvShape& c)
{
    Choice ch;
    return choose(c, ch);
}

const char* f32_mfma_kernel_name(const ConvShape& c)
{
    Choice ch;
    if (!choose(c, ch)) return nullptr;
    return use_small(c, ch) ? "conv_f32_small_kernel" : "conv_f32_mfma_kernel";
}

int launch_conv_f32_mfma(const float* x, const float* w, float* y, const ConvShape& c,
                         hipStream_t stream)
{
    Choice ch;
    if (!choose(c, ch)) return -1;
    if (use_small(c, ch)) {
        const int rc = launch_conv_f32_small(x, w, y, c, stream);
        if (rc != -1) return rc;
    }
    if (ch.grid < 1 || ch.grid > 0x7fffffff) return -1;
    MArgs args = ch.a;
    args.swz = knob(KNOB_TILE_ORDER) != 1;
    args.sync = knob(KNOB_SYNC_STAGING) == 1;
    void* params[] = {(void*)&x, (void*)&w, (void*)&y, (void*)&args};
    const dim3 grid((unsigned)ch.grid), block(64 * ch.nw);
    const hipError_t e = hipLaunchKernel(ch.f, grid, block, params, ch.lds, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return launch_status(e);
    }
    return launch_status();
}

}  // namespace im2win
