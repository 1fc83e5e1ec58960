// fp16 im2win convolution on the CDNA4 matrix cores for thin layers: few
// input channels, so the whole filter stays in LDS (fp32 accumulate; filter
// prepacked or gathered).
//
// The half-precision path of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Abstract: half
// precision on matrix hardware; Table I, cv3: 3 input channels, 64 filters
// of 7 x 7, stride 2), on the im2win property of "Im2win: Memory Efficient
// Convolution On SIMD Architectures" (Abstract): the part of a window in one
// input row is one contiguous run of that row.
//
//  * GEMM view: rows = output channels (A = filters), columns = output
//    pixels numbered over the batch (B = windows), K = (input channel c,
//    filter row kh, filter column kw) with kw padded to 8, as in the
//    row-staged kernel: a K slice of 8 is one (c, kh), for a pixel the 8
//    consecutive input columns wo*sw .. wo*sw+7 of input row ho*sh+kh. With
//    an even column stride each lane's B operand is one 4-byte-aligned
//    16-byte LDS read. Channel-interleaved slices would pad 3 channels to 8;
//    these pad 7 taps to 8.
//  * The whole contraction is one stage: a workgroup copies the filter
//    slices of its 64 output channels (direct global-to-LDS loads from the
//    prepacked filter, or gathered from w without one) and the
//    input rows of its pixels, for every input channel (through registers,
//    so rows of any width and alignment are taken), then runs all the MFMAs
//    and stores. Four waves each hold a 2 x NB tile of 32 x 32 accumulators
//    (64 channels x 32*NB pixels). With NB = 2 (256-pixel tiles, the
//    default) up to four workgroups share a CU, so some load or store while
//    others run MFMAs; the layer is bound by its fp32 output, not by the
//    matrix cores.
//  * An odd slice count gets a zero partner slice: its filter entries are
//    written as zeros and lanes 32-63 zero their B slice, and taps kw >= Wf
//    are zero in the filter and masked in B, so an infinity next to a window
//    never turns into NaN.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "knobs.hpp"

namespace im2win {

namespace {

constexpr int kThinLds = 160 * 1024;
constexpr int kCoT = 64;                  // output channels per tile
constexpr int kNW = 4;                    // waves per workgroup
constexpr int kNT = 64 * kNW;
constexpr int kMaxSlices = 64;            // filter slices (c, kh) held in LDS
constexpr int kBatch = 8;                 // row chunks a thread has in flight
constexpr uint32_t kMissT = 0xFFFFFFF0u;  // vector offset past every accepted buffer

struct ThinArgs {
    ConvShape c;
    int P;                          // pixels per tile: 32 * NB * kNW
    int co_tiles;
    int64_t px_tiles, total, tiles_per_image;
    bool aligned;                   // tiles never cross images
    int rows_max, kmax, dup, RIN;   // output rows per tile, image breaks, sh<Hf overlap, LDS rows per channel
    int RP, CH;                     // halves per LDS row (multiple of 8); its 16-byte chunks
    int S, Sp;                      // filter slices Ci*Hf; rounded up to even
    int Copad;                      // prepacked filter channels (multiple of 64)
    int chunks;                     // row chunks of a tile: Ci * RIN * CH
    int KT;                         // entries of the slice offset table
    uint32_t xoff, tab, lds_bytes;  // LDS byte offsets of the rows and the table; total
    uint32_t xbytes, ybytes, wbytes, worig;   // x, y, prepacked filter, filter in w's layout
    uint32_t mask[4];               // B dwords: halves kw >= Wf cleared
    FastDiv divWo, divHo, divCH, divRIN;
    bool swz;                       // XCD-grouped tile order
    bool sync;                      // filter copied through registers
};



// NB: 32-pixel blocks per wave (2 x NB register tiles; NB = 2 leaves room
// for four workgroups per CU, NB = 4 for two). XVEC: Wi % 8 == 0 and x
// 16-byte aligned, so a row chunk is one 16-byte load; otherwise a 16-byte
// and a 4-byte load from the dword boundary at or below it, shifted. M3:
// Wf >= 6, only the last B dword holds padded taps. WPK: the filter comes
// prepacked (wp); otherwise each workgroup gathers its slices from w.
template <int NB, bool XVEC, bool M3, bool WPK>
__global__ __launch_bounds__(kNT, 8 / NB) void conv_f16_thin_kernel(const uint16_t* __restrict__ x,
                                                               const uint4* __restrict__ wp,
                                                               const uint16_t* __restrict__ w,
                                                               float* __restrict__ y, ThinArgs a)
{
    constexpr int kNB = NB, kP = 32 * NB * kNW;
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
        q0 = img * plane + (pt - img * a.tiles_per_image) * kP;
        qend = min(q0 + kP, (img + 1) * plane);
    } else {
        q0 = pt * kP;
        qend = q0 + kP < a.total ? q0 + kP : a.total;
    }
    const int gr0 = (int)(q0 / Wo);
    const int grl = (int)((qend - 1) / Wo);
    const int n0 = (int)a.divHo.div((uint32_t)gr0);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int wave = uniform(tid >> 6);

    // Byte offset, within the rows, of each pixel's tap (c=0, kh=0, kw=0):
    // LDS row of its output row gr (tile-relative r*sh plus image breaks
    // k*dup) times the row pitch, plus its first column wo*sw.
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

    // LDS row i (of a channel) -> (image n, input row h); false if no input
    // row maps there. Segment k holds the output rows of image n0+k that
    // fall in the tile.
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

    // Filter: kilobyte m of LDS = slice m (c, kh) for the tile's 64 channels,
    // entry m*64 + j = taps kw 0..7 of w[co0 + j][c][kh][*] (zeros past Wf
    // and Co): from the prepacked filter, entries m*Copad + co0 + j, or
    // gathered from w, whose taps of slice m of channel co start at element
    // (co*Ci*Hf + m)*Wf.
    // The whole tile is one stage, so no copy overlaps an MFMA either way;
    // sync copies the filter through registers instead of loading it
    // straight into LDS.
    if (WPK && a.sync) {
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(wp, a.wbytes);
#pragma unroll 4
        for (int m = wave; m < a.S; m += kNW) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(
                r, (int)((m * a.Copad + co0 + lane) * 16), 0, 0);
            *reinterpret_cast<uint4*>(smem + (size_t)m * 1024 + 16 * lane) =
                make_uint4(v[0], v[1], v[2], v[3]);
        }
    } else if (WPK) {
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(wp, a.wbytes);
        for (int m = wave; m < a.S; m += kNW)
            lds_dma16(r, lbase + (uint32_t)m * 1024, (uint32_t)((m * a.Copad + co0 + lane) * 16));
    } else {
        // Without a prepacked filter: entry m*64 + j holds the Wf taps of
        // w[co0 + j][c][kh][*] (m = c*Hf + kh), one run of w at element
        // (co*S + m)*Wf: a 16-byte load from the dword boundary at or below
        // it (and the next dword when Wf = 8), shifted down 2 bytes when the
        // run starts between dwords, taps kw >= Wf cleared. w is read through
        // a buffer that starts at the dword boundary at or below it; an entry
        // whose loads would reach past w's end is read tap by tap. Wave v
        // takes channels 16v .. 16v+15, lane l channel 16v + l % 16 of
        // slices 4i + l / 16, so a wave's loads touch few cache lines and
        // each 8 lanes write 128 consecutive LDS bytes.
        const __amdgpu_buffer_rsrc_t r = raw_rsrc(w, a.worig);
        const uint32_t wal = (uint32_t)((uintptr_t)w & 3);
        const uint32_t wrng = a.worig + wal;
        const __amdgpu_buffer_rsrc_t ra =
            raw_rsrc(reinterpret_cast<const unsigned char*>(w) - wal, wrng);
        uint4* F = reinterpret_cast<uint4*>(smem);
        const int jc = (lane & 15) + 16 * wave;
        const int co = co0 + jc;
        constexpr int kRE = 4;   // entries per thread with loads in flight together
        for (int i0 = 0; 4 * i0 < a.S; i0 += kRE) {
            uint4 u[kRE];
            uint32_t t[kRE], sh[kRE], src[kRE];
            bool tl[kRE];
#pragma unroll
            for (int k = 0; k < kRE; ++k) {
                const int m = 4 * (i0 + k) + (lane >> 4);
                src[k] = m < a.S && co < Co ? (uint32_t)((co * a.S + m) * a.c.Wf * 2) : kMissT;
                const uint32_t sa = (src[k] + wal) & ~3u;
                tl[k] = src[k] != kMissT && sa + 20 > wrng;
                const bool hit = src[k] != kMissT && !tl[k];
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(hit ? sa : kMissT), 0, 0);
                u[k] = make_uint4(v[0], v[1], v[2], v[3]);
                t[k] = a.c.Wf == 8 ? __builtin_amdgcn_raw_buffer_load_b32(
                                         ra, (int)(hit ? sa + 16 : kMissT), 0, 0)
                                   : 0u;
                sh[k] = ((src[k] + wal) & 2u) * 8u;
            }
#pragma unroll
            for (int k = 0; k < kRE; ++k) {
                const int m = 4 * (i0 + k) + (lane >> 4);
                if (m >= a.S) continue;
                uint4 e;
                if (tl[k]) {
                    uint32_t hv[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        hv[q] = __builtin_amdgcn_raw_buffer_load_b16(
                            r, (int)(q < a.c.Wf ? src[k] + 2 * q : kMissT), 0, 0);
                    e = make_uint4(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16),
                                   hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16));
                } else {
                    e = make_uint4(__builtin_amdgcn_alignbit(u[k].y, u[k].x, sh[k]),
                                   __builtin_amdgcn_alignbit(u[k].z, u[k].y, sh[k]),
                                   __builtin_amdgcn_alignbit(u[k].w, u[k].z, sh[k]),
                                   __builtin_amdgcn_alignbit(t[k], u[k].w, sh[k]));
                }
                e.x &= a.mask[0];
                e.y &= a.mask[1];
                e.z &= a.mask[2];
                e.w &= a.mask[3];
                F[m * 64 + jc] = e;
            }
        }
    }
    if (a.Sp > a.S && wave == kNW - 1)
        reinterpret_cast<uint4*>(smem)[a.S * 64 + lane] = make_uint4(0, 0, 0, 0);
    // Slice s = (c, kh) starts (c*RIN + kh) rows into the rows; entries from
    // S on point at row 0 (their reads are unused or zeroed).
    int* T = reinterpret_cast<int*>(smem + a.tab);
    for (int j = tid; j < a.KT; j += kNT) {
        int v = 0;
        if (j < a.S) {
            const int c = j / Hf, kh = j - (j / Hf) * Hf;
            v = (c * a.RIN + kh) * a.RP * 2;
        }
        T[j] = v;
    }
    // Rows: chunk e = (cl*RIN + i)*CH + cc holds columns 8cc .. 8cc+7 of LDS
    // row i of channel cl (zeros where no input row maps and from column Wi
    // on, except in the chunk that holds column Wi - 1 of an odd-width row:
    // its halves past the row hold the next elements of x, in columns >= Wi,
    // which are only ever multiplied under the tap mask). Unaligned rows:
    // the 8 halves of a chunk are the 20 bytes from the dword boundary at or
    // below the chunk (a 16-byte and a 4-byte load, dword aligned), shifted
    // down 2 bytes where the chunk starts between dwords, through a buffer
    // that starts at the dword boundary at or below x; a chunk whose 20
    // bytes would reach past x's end (only at x's last row) takes its halves
    // one by one.
    {
        uint4* X = reinterpret_cast<uint4*>(smem + a.xoff);
        const __amdgpu_buffer_rsrc_t rx = raw_rsrc(x, a.xbytes);
        const uint32_t xa = XVEC ? 0u : (uint32_t)((uintptr_t)x & 3);
        const uint32_t rng = a.xbytes + xa;
        const __amdgpu_buffer_rsrc_t ra =
            raw_rsrc(reinterpret_cast<const unsigned char*>(x) - xa, rng);
        for (int e0 = 0; e0 < a.chunks; e0 += kBatch * kNT) {
            uint4 v[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int e = e0 + k * kNT + tid;
                uint32_t src = kMissT;
                int ncol = 0;
                if (e < a.chunks) {
                    const int row = (int)a.divCH.div((uint32_t)e);
                    const int cc = e - row * a.CH;
                    const int cl = (int)a.divRIN.div((uint32_t)row);
                    const int i = row - cl * a.RIN;
                    int n, h;
                    if (8 * cc < Wi && x_src(i, n, h)) {
                        src = (uint32_t)(((((int64_t)n * Ci + cl) * Hi + h) * Wi + 8 * cc) * 2);
                        ncol = min(8, Wi - 8 * cc);
                    }
                }
                if (XVEC) {
                    const auto u = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)src, 0, 0);
                    v[k] = make_uint4(u[0], u[1], u[2], u[3]);
                    continue;
                }
                const uint32_t sa = (src + xa) & ~3u;
                if (src != kMissT && sa + 20 > rng) {
                    uint32_t d[4] = {0, 0, 0, 0};
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        d[q >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                         rx, (int)(q < ncol ? src + 2 * q : kMissT), 0, 0)
                                     << (16 * (q & 1));
                    v[k] = make_uint4(d[0], d[1], d[2], d[3]);
                } else {
                    const bool hit = src != kMissT;
                    const auto u = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(hit ? sa : kMissT),
                                                                         0, 0);
                    const uint32_t t = __builtin_amdgcn_raw_buffer_load_b32(
                        ra, (int)(hit ? sa + 16 : kMissT), 0, 0);
                    const uint32_t sh = ((src + xa) & 2u) * 8u;
                    v[k] = make_uint4(__builtin_amdgcn_alignbit(u[1], u[0], sh),
                                      __builtin_amdgcn_alignbit(u[2], u[1], sh),
                                      __builtin_amdgcn_alignbit(u[3], u[2], sh),
                                      __builtin_amdgcn_alignbit(t, u[3], sh));
                }
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int e = e0 + k * kNT + tid;
                if (e < a.chunks) X[e] = v[k];
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's filter loads
    __syncthreads();

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
    const unsigned char* X = smem + a.xoff;
    const uint4* A = reinterpret_cast<const uint4*>(smem);
    int on0 = T[hl], on1 = T[2 + hl];
    // Pair t: slices 2t (lanes 0-31) and 2t+1 (lanes 32-63).
    auto fetch = [&](Frags& f, int t) {
        const int o = on0;
        on0 = on1;
        on1 = T[2 * t + 4 + hl];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 u = A[(2 * t + hl) * kCoT + i * 32 + l32];
            __builtin_memcpy(&f.a[i], &u, 16);
        }
        // B addresses are 4-byte aligned (even column stride, row pitch a
        // multiple of 8 halves), not 16-byte aligned: stated so, the reads
        // become aligned dword-pair reads instead of the slow unaligned form.
#pragma unroll
        for (int b = 0; b < kNB; ++b)
            __builtin_memcpy(&f.b[b], __builtin_assume_aligned(X + pb[b] + o, 4), 16);
    };
    const uint32_t m0 = a.mask[0], m1 = a.mask[1], m2 = a.mask[2], m3 = a.mask[3];
    auto mma = [&](Frags& f, uint32_t keep) {
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            uint4 u;
            __builtin_memcpy(&u, &f.b[b], 16);
            if (!M3) {
                u.x &= m0 & keep;
                u.y &= m1 & keep;
                u.z &= m2 & keep;
            } else {
                u.x &= keep;
                u.y &= keep;
                u.z &= keep;
            }
            u.w &= m3 & keep;
            __builtin_memcpy(&f.b[b], &u, 16);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                acc[i][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[i], f.b[b], acc[i][b], 0, 0, 0);
        }
    };

    const int nfull = a.S >> 1;   // pairs of two real slices
    const bool odd = (a.S & 1) != 0;
    Frags f0, f1;
    fetch(f0, 0);
    int t = 0;
    for (; t + 2 <= nfull; t += 2) {
        fetch(f1, t + 1);
        __builtin_amdgcn_sched_barrier(0);
        mma(f0, ~0u);
        __builtin_amdgcn_sched_barrier(0);
        fetch(f0, t + 2);
        __builtin_amdgcn_sched_barrier(0);
        mma(f1, ~0u);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Left: f0 = pair t.
    if (t < nfull) {
        if (odd) fetch(f1, t + 1);
        mma(f0, ~0u);
        f0 = f1;
    }
    // The last slice's zero partner: lanes 32-63 zero their B slice.
    if (odd) mma(f0, hl ? 0u : ~0u);

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

// Plans a launch; false if the shape is outside the kernel's envelope:
// fewer than 8 input channels, Ci*Hf <= 64 filter slices, Wf <= 8, an even
// column stride, LDS for the tile, tensors addressable with 32-bit buffer
// offsets. Knobs (tuning and tests): KNOB_F16_THIN < 0 turns the kernel
// off and KNOB_F16_THIN_NB picks 2 or 4 pixel blocks per wave.
bool plan(const ConvShape& c, ThinArgs& a)
{
    if (knob(KNOB_F16_THIN) < 0) return false;
    if (c.Ci >= 8 || c.Wf > 8 || c.sw % 2 != 0 || c.Hf * c.Wf > 256) return false;
    a.c = c;
    a.S = c.Ci * c.Hf;
    if (a.S > kMaxSlices) return false;
    a.Sp = (a.S + 1) & ~1;
    a.total = (int64_t)c.N * c.Ho * c.Wo;
    a.dup = std::max(0, c.Hf - c.sh);
    if ((int64_t)c.N * c.Ho > 0x7fffffff) return false;
    const int64_t plane = (int64_t)c.Ho * c.Wo;
    const int kP = a.P = 32 * kNW * (knob(KNOB_F16_THIN_NB) == 4 ? 4 : 2);
    a.rows_max = (int)std::min<int64_t>((kP - 1) / c.Wo + 2, (int64_t)c.N * c.Ho);
    a.tiles_per_image = (plane + kP - 1) / kP;
    a.aligned = (double)(a.tiles_per_image * kP) <= 1.05 * (double)plane;
    a.kmax = a.aligned || a.rows_max <= 1 ? 0 : std::min(c.N - 1, ceil_div(a.rows_max - 1, c.Ho));
    a.RIN = (a.rows_max - 1) * c.sh + c.Hf + a.kmax * a.dup;
    a.RP = ((std::max(c.Wi, (c.Wo - 1) * c.sw + 8) + 7) / 8) * 8;
    a.CH = a.RP / 8;
    const int64_t chunks = (int64_t)c.Ci * a.RIN * a.CH;
    a.KT = (a.Sp + 8 + 3) & ~3;
    a.xoff = (uint32_t)a.Sp * 1024;
    const int64_t tab = a.xoff + chunks * 16;
    // With an even slice count the A reads run one pair (2 KB) past the
    // filter: within the rows when those are that large.
    const int64_t lds = std::max<int64_t>(tab + (a.KT * 4 + 15) / 16 * 16,
                                          ((int64_t)a.Sp + (a.S % 2 == 0 ? 2 : 0)) * 1024);
    if (lds > kThinLds) return false;
    a.chunks = (int)chunks;
    a.tab = (uint32_t)tab;
    a.lds_bytes = (uint32_t)lds;
    a.Copad = ceil_div(c.Co, kCoT) * kCoT;
    a.co_tiles = a.Copad / kCoT;
    a.px_tiles = a.aligned ? (int64_t)c.N * a.tiles_per_image : (a.total + kP - 1) / kP;
    if (a.px_tiles * a.co_tiles > 0x7fffffff) return false;
    const int64_t xb = (int64_t)c.N * c.Ci * c.Hi * c.Wi * 2;
    const int64_t yb = (int64_t)c.N * c.Co * c.Ho * c.Wo * 4;
    const int64_t wb = (int64_t)a.S * a.Copad * 16;
    const int64_t wo = (int64_t)c.Co * c.Ci * c.Hf * c.Wf * 2;
    if (xb >= (int64_t)kMissT - 16 || yb >= (int64_t)kMissT || wb >= (int64_t)kMissT ||
        wo >= 0x7fffffff)
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
    a.divCH = FastDiv((uint32_t)a.CH);
    a.divRIN = FastDiv((uint32_t)a.RIN);
    a.swz = knob(KNOB_TILE_ORDER) != 1;
    a.sync = knob(KNOB_SYNC_STAGING) == 1;
    return true;
}

template <int NB, bool XVEC, bool M3, bool WPK>
int launch_t(const uint16_t* x, const uint4* wp, const uint16_t* w, float* y, const ThinArgs& a,
             hipStream_t stream)
{
    ensure_lds_limit((const void*)conv_f16_thin_kernel<NB, XVEC, M3, WPK>, kThinLds);
    hipLaunchKernelGGL((conv_f16_thin_kernel<NB, XVEC, M3, WPK>),
                       dim3((unsigned)(a.px_tiles * a.co_tiles)), dim3(kNT), a.lds_bytes, stream, x,
                       wp, w, y, a);
    return launch_status();
}

template <int NB, bool WPK>
int launch_nb(const uint16_t* x, const uint4* wp, const uint16_t* w, float* y, const ThinArgs& a,
              bool xvec, hipStream_t stream)
{
    const bool m3 = a.c.Wf >= 6;
    if (xvec) return m3 ? launch_t<NB, true, true, WPK>(x, wp, w, y, a, stream)
                        : launch_t<NB, true, false, WPK>(x, wp, w, y, a, stream);
    return m3 ? launch_t<NB, false, true, WPK>(x, wp, w, y, a, stream)
              : launch_t<NB, false, false, WPK>(x, wp, w, y, a, stream);
}

}  // namespace

bool f16_thin_applies(const ConvShape& c)
{
    ThinArgs a;
    return plan(c, a);
}

int launch_conv_f16_thin(const uint16_t* x, const void* wp, const uint16_t* w, float* y,
                         const ConvShape& c, hipStream_t stream)
{
    ThinArgs a;
    if (!plan(c, a)) return -1;
    if ((uintptr_t)wp % 16 != 0) return -1;
    const uint4* w4 = static_cast<const uint4*>(wp);
    const bool xvec = c.Wi % 8 == 0 && (uintptr_t)x % 16 == 0;
    const bool nb2 = a.P == 32 * kNW * 2;
    if (w4) return nb2 ? launch_nb<2, true>(x, w4, w, y, a, xvec, stream)
                       : launch_nb<4, true>(x, w4, w, y, a, xvec, stream);
    return nb2 ? launch_nb<2, false>(x, w4, w, y, a, xvec, stream)
               : launch_nb<4, false>(x, w4, w, y, a, xvec, stream);
}

}  // namespace im2win
