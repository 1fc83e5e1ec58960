// fp32 im2win convolution on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The single-precision path of "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (Section III:
// the convolution as dot products of filter rows with im2win windows) for
// one MI355X. fp32 products and fp32 accumulation, as on the vector ALUs, but
// at the matrix-core rate (twice the unpacked vector FMA rate):
//
//  * GEMM view: rows = output channels (A = filters), columns = output
//    pixels (B = windows), K = (input channel, kh, kw) in the filter's own
//    memory order. Pixels are numbered over the whole batch,
//    q = (n*Ho + ho)*Wo + wo. A workgroup of four waves owns 32*WCO channels
//    and 128 consecutive pixels; wave v owns pixels 32v..32v+31 of the tile
//    and all 32*WCO channels (WCO MFMA tiles, AGPR accumulators).
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
//  * Small problems split K over workgroups and add their partial sums into
//    the zero-filled output with hardware float atomics.
#include <algorithm>
#include <cstdlib>

#include "common.hpp"
#include "kernels.hpp"

namespace im2win {

namespace {

constexpr int kMaxLds = 160 * 1024;
constexpr int kNT = 256;      // four waves
constexpr int kP = 128;       // pixels per tile: 32 per wave
constexpr int kRPW = 8;       // input rows per wave and stage (32 per workgroup)
constexpr uint32_t kMaxBuf = 0xFFFFFFF0u;   // buffer ranges are 32-bit

struct MArgs {
    ConvShape c;
    int co_tiles, ksplit, spk;        // channel tiles; K splits; stages per split
    int64_t px_tiles, total, tiles_per_image;
    bool aligned;                     // tiles never cross images
    int rows_max, kmax, dup, RIN;     // output rows per tile, image breaks, s<Hf overlap, LDS rows
    int HW, CB, nstages, KSP;         // taps; channels per stage; stages; filter row pitch (odd)
    int NU, RS, CSX, xent;            // entries per phase, per row (s*NU), per channel; total
    uint32_t ybytes;
    FastDiv divWo, divHo, divS;
};

// Raw buffer resource over [base, base + bytes): loads at soffset + voffset
// + offset >= bytes return 0 (the scalar offset counts in the range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

template <int WCO, int XCH, int WCH>
__global__ __launch_bounds__(kNT) void conv_f32_mfma_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            float* __restrict__ y, MArgs a)
{
    constexpr int COT = 32 * WCO;
    constexpr int WRW = COT / 4;   // filter rows per wave and stage

    extern __shared__ __align__(16) float lds[];
    float* X = lds;
    float* Wl = lds + a.xent;

    const int Ci = a.c.Ci, Hi = a.c.Hi, Wi = a.c.Wi, Co = a.c.Co, s = a.c.s;
    const int Ho = a.c.Ho, Wo = a.c.Wo, Hf = a.c.Hf, Wf = a.c.Wf;
    const int HW = a.HW, RS = a.RS, NU = a.NU, KSP = a.KSP, RIN = a.RIN, CB = a.CB;

    // blockIdx.x = (pixel tile * ksplit + split) * co_tiles + channel tile
    const int co_t = (int)(blockIdx.x % a.co_tiles);
    const int rest = (int)(blockIdx.x / a.co_tiles);
    const int ksi = rest % a.ksplit;
    const int64_t pt = rest / a.ksplit;
    const int co0 = co_t * COT;
    const int st0 = ksi * a.spk, st1 = min(a.nstages, st0 + a.spk);
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

    // This lane's pixel: entry of its tap (0, 0) in a channel's LDS rows
    // (row of output row gr: tile-relative r*s plus image breaks k*dup).
    const int64_t qme = q0 + wave * 32 + l32;
    int xb;
    {
        const int64_t q = qme < qend ? qme : qend - 1;
        const int gr = (int)a.divWo.div((uint32_t)(q - (int64_t)gr0 * Wo)) + gr0;
        const int wo = (int)(q - (int64_t)gr * Wo);
        const int k = (int)a.divHo.div((uint32_t)gr) - n0;
        xb = ((gr - gr0) * s + k * a.dup) * RS + wo;
    }
    const int abase = l32 * KSP + hl;   // A: channel l32 of each block, K index 2t + hl

    floatx16_t acc[WCO];
#pragma unroll
    for (int i = 0; i < WCO; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

    // LDS row i -> (image n, input row h); false if no input row maps there.
    auto x_src = [&](int i, int& n, int& h) -> bool {
        for (int k = 0; k <= a.kmax; ++k) {
            const int nk = n0 + k;
            const int first = max(gr0, nk * Ho), last = min(grl, nk * Ho + Ho - 1);
            if (first > last) break;
            const int S = (first - gr0) * s + k * a.dup;
            const int span = (last - first) * s + Hf;
            if (i >= S && i < S + span) {
                n = nk;
                h = (first - nk * Ho) * s + (i - S);
                return true;
            }
        }
        return false;
    };

    // Staging geometry, fixed for the tile. Wave v stages LDS rows
    // r = v + 4*ii of a stage (channel r / RIN, row r % RIN), its lanes taking
    // columns lane + 64*cc; the row's byte offset in x is the scalar offset of
    // the load, the column the vector offset, and the buffer ends where the
    // row does, so columns >= Wi read 0.
    uint32_t xrow[kRPW];
    uint32_t xvalid = 0;
#pragma unroll
    for (int ii = 0; ii < kRPW; ++ii) {
        const int r = wave + 4 * ii;
        const int cl = r / RIN, i = r - (r / RIN) * RIN;
        int n = 0, h = 0;
        xrow[ii] = 0;
        if (cl < CB && x_src(i, n, h)) {
            xrow[ii] = (uint32_t)(((((int64_t)n * Ci + cl) * Hi + h) * Wi) * 4);
            xvalid |= 1u << ii;
        }
    }
    const uint32_t lane4 = (uint32_t)lane * 4;
    int xdst[XCH];   // LDS entry of column lane + 64*cc within a row; -1 past Wi
#pragma unroll
    for (int cc = 0; cc < XCH; ++cc) {
        const int col = lane + 64 * cc;
        const int u = (int)a.divS.div((uint32_t)col);
        xdst[cc] = col < Wi ? (col - u * s) * NU + u : -1;
    }

    float xv[kRPW][XCH];
    float wv[WRW][WCH];
    const uint32_t rowb = (uint32_t)Wi * 4;
    const uint32_t wpitch = (uint32_t)Ci * HW * 4;   // bytes between filters

    auto load_stage = [&](int st) {
        const int ci0 = st * CB, cbs = min(CB, Ci - ci0);
        const uint32_t cofs = (uint32_t)ci0 * Hi * Wi * 4;
#pragma unroll
        for (int ii = 0; ii < kRPW; ++ii) {
            if (((xvalid >> ii) & 1u) && wave + 4 * ii < cbs * RIN) {
                const uint32_t so = xrow[ii] + cofs;
                const __amdgpu_buffer_rsrc_t xr = buf(x, so + rowb);
#pragma unroll
                for (int cc = 0; cc < XCH; ++cc)
                    xv[ii][cc] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        xr, (int)(lane4 + 256 * cc), (int)so, 0));
            }
        }
        // Filters co0 + co, channels ci0 .. ci0 + cbs - 1: cbs*HW contiguous
        // taps each; taps past that read as zero (the odd-K pad entry).
        const float* wst = w + ((int64_t)co0 * Ci + ci0) * HW;
        const uint32_t wlen = (uint32_t)(cbs * HW * 4);
#pragma unroll
        for (int i = 0; i < WRW; ++i) {
            const int co = wave + 4 * i;
            if (co0 + co < Co) {
                const uint32_t so = (uint32_t)co * wpitch;
                const __amdgpu_buffer_rsrc_t wr = buf(wst, so + wlen);
#pragma unroll
                for (int jc = 0; jc < WCH; ++jc)
                    wv[i][jc] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        wr, (int)(lane4 + 256 * jc), (int)so, 0));
            }
        }
    };
    auto store_stage = [&](int st) {
        const int ci0 = st * CB, cbs = min(CB, Ci - ci0);
#pragma unroll
        for (int ii = 0; ii < kRPW; ++ii) {
            const int r = wave + 4 * ii;
            if (((xvalid >> ii) & 1u) && r < cbs * RIN) {
                float* row = X + r * RS;
#pragma unroll
                for (int cc = 0; cc < XCH; ++cc)
                    if (xdst[cc] >= 0) row[xdst[cc]] = xv[ii][cc];
            }
        }
#pragma unroll
        for (int i = 0; i < WRW; ++i) {
            const int co = wave + 4 * i;
            if (co0 + co < Co) {
                float* row = Wl + co * KSP;
#pragma unroll
                for (int jc = 0; jc < WCH; ++jc)
                    if (lane + 64 * jc < KSP) row[lane + 64 * jc] = wv[i][jc];
            }
        }
    };

    // K walk in filter order (channel cl, kh, kw); the LDS offset of an index
    // from the pixel's tap (0, 0) of channel 0 is cl*CSX + kh*RS +
    // (kw % s)*NU + kw / s. Uniform (scalar unit), no divisions.
    struct Tap {
        int cl, kh, kw, ph, u;
    };
    auto tap_off = [&](const Tap& t) { return t.cl * a.CSX + t.kh * RS + t.ph * NU + t.u; };
    auto tap_next = [&](Tap& t) {
        if (++t.kw == Wf) {
            t.kw = 0; t.ph = 0; t.u = 0;
            if (++t.kh == Hf) {
                t.kh = 0; ++t.cl;
            }
        } else if (++t.ph == s) {
            t.ph = 0; ++t.u;
        }
    };
    struct Frags {
        float a[WCO], b;
    };
    auto fetch = [&](Frags& f, int offA, int offB, int kk) {
        const int off = hl ? offB : offA;
        f.b = X[xb + off];
#pragma unroll
        for (int i = 0; i < WCO; ++i) f.a[i] = Wl[abase + i * 32 * KSP + kk];
    };
    auto mma = [&](const Frags& f) {
#pragma unroll
        for (int i = 0; i < WCO; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i], f.b, acc[i], 0, 0, 0);
    };

    load_stage(st0);
    store_stage(st0);
    __syncthreads();
    for (int st = st0; st < st1; ++st) {
        if (st + 1 < st1) load_stage(st + 1);
        const int ks = min(CB, Ci - st * CB) * HW;
        const int nfull = ks >> 1;   // pairs with two real K indices
        Tap ta = {0, 0, 0, 0, 0};
        auto fetch_pair = [&](Frags& f, int t) {
            Tap tb = ta;
            tap_next(tb);
            fetch(f, tap_off(ta), tap_off(tb), 2 * t);
            ta = tb;
            tap_next(ta);
        };
        // Pair t+1 is read from LDS while the MFMAs of pair t run.
        Frags f0, f1;
        int t = 0;
        if (t < nfull) fetch_pair(f0, t);
        for (; t + 2 <= nfull; t += 2) {
            fetch_pair(f1, t + 1);
            mma(f0);
            if (t + 2 < nfull) fetch_pair(f0, t + 2);
            mma(f1);
        }
        if (t < nfull) {
            mma(f0);
            ++t;
        }
        if (ks & 1) {
            // Last K index with a zero partner: filter entry ks is zero and
            // lanes 32-63 zero their window value.
            const int off = tap_off(ta);
            fetch(f0, off, off, 2 * nfull);
            f0.b = hl ? 0.f : f0.b;
            mma(f0);
        }
        if (st + 1 < st1) {
            __syncthreads();
            store_stage(st + 1);
            __syncthreads();
        }
    }

    // Output: lane holds pixel l32 of its block and channels
    // 8*(r/4) + 4*hl + r%4 of each 32-channel block.
    const int64_t plane = (int64_t)Ho * Wo;
    const bool qok = qme < qend;
    const int64_t q = qok ? qme : qend - 1;
    const int gr = (int)(q / Wo);
    const int wo = (int)(q - (int64_t)gr * Wo);
    const int n = (int)a.divHo.div((uint32_t)gr), ho = gr - n * Ho;
    const bool all_co = co0 + COT <= Co;
    if (a.ksplit == 1) {
        // Byte offset = per-lane part (image, pixel, 4*hl channels) + uniform
        // part (channel block row).
        const __amdgpu_buffer_rsrc_t yb = buf(y, a.ybytes);
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
    } else {
        float* yp = y + (((int64_t)n * Co + 4 * hl) * plane + (int64_t)ho * Wo + wo);
#pragma unroll
        for (int i = 0; i < WCO; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int cu = co0 + i * 32 + 8 * (r >> 2) + (r & 3);
                if (qok && (all_co || cu + 4 * hl < Co))
                    unsafeAtomicAdd(yp + (int64_t)cu * plane, acc[i][r]);
            }
    }
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ y, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = 0.f;
}

int env_int(const char* name, int dflt)
{
    const char* v = std::getenv(name);
    return v && *v ? std::atoi(v) : dflt;
}

// Plans the launch; false if the shape is outside the kernel's envelope.
bool plan(const ConvShape& c, MArgs& a, int& wco, int& xch, int& wch)
{
    a.c = c;
    a.HW = c.Hf * c.Wf;
    a.total = (int64_t)c.N * c.Ho * c.Wo;
    a.dup = std::max(0, c.Hf - c.s);
    if ((int64_t)c.N * c.Ho > 0x7fffffff) return false;
    xch = ceil_div(c.Wi, 64);
    if (xch == 3) xch = 4;
    if (xch > 4) return false;
    if (a.HW > 254) return false;

    // Channel tile: least padding, then the widest.
    wco = 1;
    int best = 1 << 30;
    for (int cand = 4; cand >= 1; --cand) {
        const int waste = ceil_div(c.Co, 32 * cand) * 32 * cand - c.Co;
        if (waste < best) {
            best = waste;
            wco = cand;
        }
    }
    wco = env_int("IM2WIN_F32_WCO", wco);
    if (wco < 1 || wco > 4) return false;
    const int cot = 32 * wco;

    a.NU = ceil_div(c.Wi, c.s);
    a.RS = c.s * a.NU;
    const int64_t plane = (int64_t)c.Ho * c.Wo;
    a.rows_max = (kP - 1) / c.Wo + 2;
    a.tiles_per_image = (plane + kP - 1) / kP;
    a.aligned = c.N == 1 || (double)(a.tiles_per_image * kP) <= 1.05 * (double)plane;
    a.kmax = a.aligned || a.rows_max <= 1 ? 0 : ceil_div(a.rows_max - 1, c.Ho);
    a.RIN = (a.rows_max - 1) * c.s + c.Hf + a.kmax * a.dup;
    if (a.RIN > 4 * kRPW) return false;
    a.CSX = a.RIN * a.RS;

    // Channels per stage: fill the row slots, keep the filter rows within
    // the register prefetch (WRW x WCH loads) and the LDS budget.
    auto ksp_of = [&](int cb) { return ((cb * a.HW + 1) & ~1) + 1; };
    auto wch_of = [&](int cb) {
        const int v = ceil_div(ksp_of(cb), 64);
        return v == 3 ? 4 : v;
    };
    auto lds_of = [&](int cb) { return ((int64_t)cb * a.CSX + (int64_t)cot * ksp_of(cb)) * 4; };
    int cb = std::min(c.Ci, (4 * kRPW) / a.RIN);
    while (cb > 1 && (ksp_of(cb) > 256 || wco * wch_of(cb) > 8 || lds_of(cb) > 80 * 1024)) --cb;
    cb = std::max(1, std::min(cb, env_int("IM2WIN_F32_CB", cb)));
    if (ksp_of(cb) > 256 || wco * wch_of(cb) > 8 || lds_of(cb) > kMaxLds) return false;
    a.CB = cb;
    a.KSP = ksp_of(cb);
    wch = wch_of(cb);
    a.xent = cb * a.CSX;
    a.nstages = ceil_div(c.Ci, cb);

    a.co_tiles = ceil_div(c.Co, cot);
    a.px_tiles = a.aligned ? (int64_t)c.N * a.tiles_per_image : (a.total + kP - 1) / kP;
    // Split K when there are too few tiles to fill the chip.
    const int64_t base = a.px_tiles * a.co_tiles;
    int ksplit = 1;
    if (base < 384 && a.nstages > 1) ksplit = (int)std::min<int64_t>(a.nstages, (512 + base - 1) / base);
    ksplit = std::max(1, std::min(a.nstages, env_int("IM2WIN_F32_KSPLIT", ksplit)));
    a.spk = ceil_div(a.nstages, ksplit);
    a.ksplit = ceil_div(a.nstages, a.spk);
    if (base * a.ksplit > 0x7fffffff) return false;

    // Scalar offsets and buffer ranges are 32-bit.
    const int64_t xb = (int64_t)c.N * c.Ci * c.Hi * c.Wi * 4;
    const int64_t yb = (int64_t)c.N * c.Co * c.Ho * c.Wo * 4;
    const int64_t wb = (int64_t)c.Co * c.Ci * a.HW * 4;
    if (xb >= (int64_t)kMaxBuf || yb >= (int64_t)kMaxBuf || wb >= (int64_t)kMaxBuf) return false;
    a.ybytes = (uint32_t)yb;
    a.divWo = FastDiv((uint32_t)c.Wo);
    a.divHo = FastDiv((uint32_t)c.Ho);
    a.divS = FastDiv((uint32_t)c.s);
    return true;
}

template <int WCO, int XCH, int WCH>
int launch_t(const float* x, const float* w, float* y, const MArgs& a, hipStream_t stream)
{
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute((const void*)conv_f32_mfma_kernel<WCO, XCH, WCH>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        attr = true;
    }
    const size_t lds = ((size_t)a.xent + (size_t)32 * WCO * a.KSP) * 4;
    hipLaunchKernelGGL((conv_f32_mfma_kernel<WCO, XCH, WCH>),
                       dim3((unsigned)(a.px_tiles * a.co_tiles * a.ksplit)), dim3(kNT), lds,
                       stream, x, w, y, a);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <int WCO, int XCH>
int launch_x(const float* x, const float* w, float* y, const MArgs& a, int wch,
             hipStream_t stream)
{
    if (wch == 1) return launch_t<WCO, XCH, 1>(x, w, y, a, stream);
    if (wch == 2) return launch_t<WCO, XCH, 2>(x, w, y, a, stream);
    if (WCO <= 2 && wch == 4) return launch_t<WCO, XCH, (WCO <= 2 ? 4 : 1)>(x, w, y, a, stream);
    return -1;
}

template <int WCO>
int launch_w(const float* x, const float* w, float* y, const MArgs& a, int xch, int wch,
             hipStream_t stream)
{
    if (xch == 1) return launch_x<WCO, 1>(x, w, y, a, wch, stream);
    if (xch == 2) return launch_x<WCO, 2>(x, w, y, a, wch, stream);
    if (xch == 4) return launch_x<WCO, 4>(x, w, y, a, wch, stream);
    return -1;
}

}  // namespace

int launch_conv_f32_mfma(const float* x, const float* w, float* y, const ConvShape& c,
                         hipStream_t stream)
{
    MArgs a;
    int wco, xch, wch;
    if (!plan(c, a, wco, xch, wch)) return -1;
    if (a.ksplit > 1) {
        // Partial sums are added into y: clear it first (a kernel, not a
        // memset node, so the call stays capturable).
        const int64_t n = (int64_t)c.N * c.Co * c.Ho * c.Wo;
        const int64_t blocks = (n + 255) / 256;
        if (blocks > 0x7fffffff) return -1;
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y, n);
    }
    switch (wco) {
    case 1: return launch_w<1>(x, w, y, a, xch, wch, stream);
    case 2: return launch_w<2>(x, w, y, a, xch, wch, stream);
    case 3: return launch_w<3>(x, w, y, a, xch, wch, stream);
    case 4: return launch_w<4>(x, w, y, a, xch, wch, stream);
    }
    return -1;
}

}  // namespace im2win
