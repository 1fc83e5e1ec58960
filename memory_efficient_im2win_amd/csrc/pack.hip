// im2win transform as an HBM-bound bit copy.
//
// The transform of "Im2win: Memory Efficient Convolution On SIMD
// Architectures" (Abstract): each row of dot-product windows (image n,
// channel ci, output row ho) becomes one row holding the Hf input rows
// ho*sh .. ho*sh+Hf-1 (sh: the row stride), column by column:
//     ws[n][ci][ho][w*Hf + kh] = x[n][ci][ho*sh + kh][w]
//
// One workgroup produces R consecutive im2win rows of one (n, ci) plane, i.e.
// one contiguous stretch of ws. It first copies the (R-1)*sh + Hf input rows
// those im2win rows draw from into LDS (each input row is read from HBM once
// per workgroup even when windows overlap), then writes its stretch of ws
// with 16-byte stores; the ragged head and tail of the stretch, where ws is
// not 16-byte aligned, are written element by element. Reads are 16-byte
// vectors too, with the same head/tail treatment.
#include "common.hpp"
#include "kernels.hpp"

namespace im2win {

namespace {

constexpr int kPackThreads = 256;

struct PackArgs {
    int Hi, Wi, Hf, sh, Ho;
    int R;              // im2win rows per workgroup
    int chunks;         // workgroups per (n, ci) plane = ceil(Ho / R)
    uint32_t L;         // im2win row length Wi * Hf
    FastDiv divL, divHf;
};

template <typename T>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const T* __restrict__ x,
                                                            T* __restrict__ ws, PackArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int V = 16 / sizeof(T);  // elements per 16-byte vector

    const int64_t b = blockIdx.x;
    const int64_t plane = b / a.chunks;
    const int chunk = (int)(b - plane * a.chunks);
    const int ho0 = chunk * a.R;
    const int nr = min(a.R, a.Ho - ho0);
    const int r0 = ho0 * a.sh;
    const int nrows = (nr - 1) * a.sh + a.Hf;

    // ---- input rows [r0, r0 + nrows) of the plane -> LDS ----------------
    const T* src = x + (plane * a.Hi + r0) * (int64_t)a.Wi;
    const int nin = nrows * a.Wi;
    const uintptr_t gs = (uintptr_t)src;
    const int head = (int)((gs & 15u) / sizeof(T));   // elements before the 16-B boundary
    T* lds = reinterpret_cast<T*>(smem) + head;       // lds[i] <-> src[i], same alignment mod 16
    {
        const int first_vec = head == 0 ? 0 : V - head;  // first element on a 16-B boundary
        const int nvec = nin > first_vec ? (nin - first_vec) / V : 0;
        const uint4* gv = reinterpret_cast<const uint4*>(src + first_vec);
        uint4* lv = reinterpret_cast<uint4*>(lds + first_vec);
        for (int i = threadIdx.x; i < nvec; i += kPackThreads)
            lv[i] = gv[i];
        const int tail0 = first_vec + nvec * V;
        const int nhead = min(first_vec, nin);
        for (int i = threadIdx.x; i < nhead; i += kPackThreads)
            lds[i] = src[i];
        for (int i = tail0 + threadIdx.x; i < nin; i += kPackThreads)
            lds[i] = src[i];
    }
    __syncthreads();

    // ---- LDS -> ws stretch [(plane*Ho + ho0) * L, + nr*L) ------------------
    T* dst = ws + (plane * a.Ho + ho0) * (int64_t)a.L;
    const int nout = nr * (int)a.L;
    const int ohead = (int)(((uintptr_t)dst & 15u) / sizeof(T));
    const int first_vec = ohead == 0 ? 0 : V - ohead;
    const int nvec = nout > first_vec ? (nout - first_vec) / V : 0;

    // Source of stretch element e: im2win row hol = e / L, r = e % L,
    // column w = r / Hf, tap kh = r % Hf  ->  lds[(hol*sh + kh)*Wi + w].
    auto src_index = [&](uint32_t e, int& hol, int& w, int& kh) {
        hol = (int)a.divL.div(e);
        const uint32_t r = e - (uint32_t)hol * a.L;
        w = (int)a.divHf.div(r);
        kh = (int)(r - (uint32_t)w * a.Hf);
    };

    uint4* dv = reinterpret_cast<uint4*>(dst + first_vec);
    for (int i = threadIdx.x; i < nvec; i += kPackThreads) {
        int hol, w, kh;
        src_index((uint32_t)(first_vec + i * V), hol, w, kh);
        T v[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
            v[j] = lds[(hol * a.sh + kh) * a.Wi + w];
            if (++kh == a.Hf) {
                kh = 0;
                if (++w == a.Wi) { w = 0; ++hol; }
            }
        }
        uint4 pk;
        __builtin_memcpy(&pk, v, 16);
        dv[i] = pk;
    }
    const int nhead = min(first_vec, nout);
    const int tail0 = nhead + nvec * V;
    for (int e = threadIdx.x; e < nhead + (nout - tail0); e += kPackThreads) {
        const int idx = e < nhead ? e : tail0 + (e - nhead);
        int hol, w, kh;
        src_index((uint32_t)idx, hol, w, kh);
        dst[idx] = lds[(hol * a.sh + kh) * a.Wi + w];
    }
}

// Fallback for rows too long to stage in LDS: one element per thread,
// gathered straight from x.
template <typename T>
__global__ __launch_bounds__(kPackThreads) void pack_gather_kernel(const T* __restrict__ x,
                                                                   T* __restrict__ ws,
                                                                   PackArgs a, int64_t total)
{
    const int64_t e = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    if (e >= total) return;
    const int64_t row = e / a.L;                       // (plane, ho)
    const int r = (int)(e - row * a.L);
    const int64_t plane = row / a.Ho;
    const int ho = (int)(row - plane * a.Ho);
    const int w = r / a.Hf, kh = r - (r / a.Hf) * a.Hf;
    ws[e] = x[(plane * a.Hi + (int64_t)ho * a.sh + kh) * a.Wi + w];
}

}  // namespace

int launch_pack(const void* x, void* ws, int N, int Ci, int Hi, int Wi, int Hf, int sh,
                int Ho, int elem_bytes, hipStream_t stream)
{
    PackArgs a;
    a.Hi = Hi; a.Wi = Wi; a.Hf = Hf; a.sh = sh; a.Ho = Ho;
    a.L = (uint32_t)Wi * (uint32_t)Hf;
    // Aim for ~32 KiB written per workgroup, with the staged input rows
    // bounded to 48 KiB of LDS.
    const int64_t row_bytes = (int64_t)a.L * elem_bytes;
    int R = (int)std::max<int64_t>(1, (32 * 1024) / std::max<int64_t>(row_bytes, 1));
    R = std::min(R, Ho);
    while (R > 1 && ((int64_t)((R - 1) * sh + Hf) * Wi * elem_bytes + 16) > 48 * 1024) --R;
    a.R = R;
    a.chunks = ceil_div(Ho, R);
    a.divL = FastDiv(a.L);
    a.divHf = FastDiv((uint32_t)Hf);
    const int64_t blocks = (int64_t)N * Ci * a.chunks;
    const size_t lds = (size_t)((R - 1) * sh + Hf) * Wi * elem_bytes + 16;
    if (blocks <= 0 || blocks > 0x7fffffff) return -1;
    if (lds > 64 * 1024) {
        const int64_t total = (int64_t)N * Ci * Ho * (int64_t)a.L;
        const int64_t gb = (total + kPackThreads - 1) / kPackThreads;
        if (gb > 0x7fffffff) return -1;
        if (elem_bytes == 2)
            hipLaunchKernelGGL(pack_gather_kernel<uint16_t>, dim3((unsigned)gb), dim3(kPackThreads),
                               0, stream, (const uint16_t*)x, (uint16_t*)ws, a, total);
        else
            hipLaunchKernelGGL(pack_gather_kernel<uint32_t>, dim3((unsigned)gb), dim3(kPackThreads),
                               0, stream, (const uint32_t*)x, (uint32_t*)ws, a, total);
        return launch_status();
    }
    if (elem_bytes == 2)
        hipLaunchKernelGGL(pack_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kPackThreads), lds,
                           stream, (const uint16_t*)x, (uint16_t*)ws, a);
    else
        hipLaunchKernelGGL(pack_kernel<uint32_t>, dim3((unsigned)blocks), dim3(kPackThreads), lds,
                           stream, (const uint32_t*)x, (uint32_t*)ws, a);
    return launch_status();
}

}  // namespace im2win
