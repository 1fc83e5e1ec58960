// C ABI of the im2win library: argument checks, workspace/mode selection and
// kernel dispatch. Declarations and the contract are in include/im2win.h.
#include <algorithm>
#include <map>
#include <mutex>
#include <stdint.h>
#include <utility>

#include "im2win.h"
#include "kernels.hpp"
#include "knobs.hpp"

namespace {

using im2win::ConvShape;

constexpr int64_t kMax32 = 0x7fffffff;

// Derives Ho, Wo and checks every limit of the contract (sh, sw: row and
// column strides).
bool check_shape(int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw, int* Ho,
                 int* Wo)
{
    if (N < 1 || Ci < 1 || Hi < 1 || Wi < 1 || Co < 1 || Hf < 1 || Wf < 1) return false;
    if (sh < 1 || sw < 1) return false;
    if (Hf > Hi || Wf > Wi) return false;
    const int ho = (Hi - Hf) / sh + 1, wo = (Wi - Wf) / sw + 1;
    if ((int64_t)Ci * Hi * Wi > kMax32) return false;
    if ((int64_t)Co * ho * wo > kMax32) return false;
    if ((int64_t)Ci * ho * Wi * Hf > kMax32) return false;
    if ((int64_t)Co * Ci * Hf * Wf > kMax32) return false;
    if (Ho) *Ho = ho;
    if (Wo) *Wo = wo;
    return true;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int status_of(int rc)
{
    if (rc == 0) return IM2WIN_OK;
    if (rc == -1) return IM2WIN_EINVAL;
    return IM2WIN_ELAUNCH;
}

thread_local hipError_t g_last_error = hipSuccess;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Bytes of one image's im2win rows (the unit of the materialised mode).
size_t im2win_image_bytes(const ConvShape& c, size_t elem)
{
    return (size_t)c.Ci * c.Ho * c.Wi * c.Hf * elem;
}

// Shared driver of both precisions (the workspace contract of
// conv2d_im2win_fp32 / _fp16). T is the element type of x, w and ws.
template <typename T>
int conv_driver(const T* x, const T* w, float* y, void* ws, size_t ws_bytes, int N, int Ci, int Hi,
                int Wi, int Co, int Hf, int Wf, int sh, int sw, hipStream_t stream,
                int (*fused)(const T*, const T*, const void*, float*, const ConvShape&, hipStream_t),
                int (*from_ws)(const T*, const T*, const T*, float*, const ConvShape&, hipStream_t),
                int (*generic)(const T*, const T*, const T*, float*, const ConvShape&, hipStream_t))
{
    int Ho, Wo;
    if (!x || !w || !y) return IM2WIN_EINVAL;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return IM2WIN_EINVAL;
    if (!aligned(x, sizeof(T)) || !aligned(w, sizeof(T)) || !aligned(y, sizeof(float)))
        return IM2WIN_EINVAL;
    const ConvShape c{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo};
    if (ws == nullptr) {
        if (ws_bytes != 0) return IM2WIN_EWORKSPACE;
        int rc = fused(x, w, nullptr, y, c, stream);
        if (rc == -1) rc = generic(x, nullptr, w, y, c, stream);
        return status_of(rc);
    }
    if (!aligned(ws, 16)) return IM2WIN_EINVAL;
    // Materialised: the im2win tensor of as many images as fit, chunk by
    // chunk, at the start of the workspace.
    const size_t per_image = im2win_image_bytes(c, sizeof(T));
    if (ws_bytes < per_image) return IM2WIN_EWORKSPACE;
    const T* ims = static_cast<const T*>(ws);
    const int chunk = (int)std::min<size_t>((size_t)N, ws_bytes / per_image);
    const int64_t x_img = (int64_t)Ci * Hi * Wi, y_img = (int64_t)Co * Ho * Wo;
    for (int n0 = 0; n0 < N; n0 += chunk) {
        const int nc = std::min(chunk, N - n0);
        int rc = im2win::launch_pack(x + n0 * x_img, ws, nc, Ci, Hi, Wi, Hf, sh, Ho,
                                     (int)sizeof(T), stream);
        if (rc != 0) return status_of(rc);
        ConvShape cc = c;
        cc.N = nc;
        rc = from_ws(x + n0 * x_img, ims, w, y + n0 * y_img, cc, stream);
        if (rc == -1) rc = generic(x + n0 * x_img, ims, w, y + n0 * y_img, cc, stream);
        if (rc != 0) return status_of(rc);
    }
    return IM2WIN_OK;
}

// Adapters to the driver's signatures.
// fp32 fused: the matrix-core kernel where the shape fits its envelope,
// else the vector-ALU kernel. KNOB_F32_VALU = 1 selects the latter always.
int f32_fused(const float* x, const float* w, const void*, float* y, const ConvShape& c,
              hipStream_t st)
{
    if (im2win::knob(im2win::KNOB_F32_VALU) != 1) {
        const int rc = im2win::launch_conv_f32_mfma(x, w, y, c, st);
        if (rc != -1) return rc;
    }
    return im2win::launch_conv_f32(x, nullptr, w, y, c, st);
}
int f32_from_ws(const float* x, const float* ws, const float* w, float* y, const ConvShape& c,
                hipStream_t st)
{
    return im2win::launch_conv_f32(x, ws, w, y, c, st);
}
int f32_generic(const float* x, const float* ws, const float* w, float* y, const ConvShape& c,
                hipStream_t st)
{
    return im2win::launch_conv_generic_f32(x, ws, w, y, c, st);
}
int f16_from_ws(const uint16_t* x, const uint16_t* ws, const uint16_t* w, float* y,
                const ConvShape& c, hipStream_t st)
{
    const int rc = im2win::launch_conv_f16_ws(ws, w, y, c, st);
    if (rc != -1) return rc;
    return im2win::launch_conv_f16(x, ws, w, y, c, st);
}
int f16_generic(const uint16_t* x, const uint16_t* ws, const uint16_t* w, float* y,
                const ConvShape& c, hipStream_t st)
{
    return im2win::launch_conv_generic_f16(x, ws, w, y, c, st);
}

// fp16 fused with the filter prepacked per call into fws (fws_bytes >=
// im2win::f16_filter_pack_bytes), or gathered in the kernel (fws NULL).
int f16_fused_driver(const uint16_t* x, const uint16_t* w, float* y, void* fws, size_t fws_bytes,
                     int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw,
                     hipStream_t stream)
{
    int Ho, Wo;
    if (!x || !w || !y) return IM2WIN_EINVAL;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return IM2WIN_EINVAL;
    if (!aligned(x, 2) || !aligned(w, 2) || !aligned(y, 4)) return IM2WIN_EINVAL;
    const ConvShape c{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo};
    if (fws == nullptr) {
        if (fws_bytes != 0) return IM2WIN_EWORKSPACE;
        int rc = im2win::launch_conv_f16_fused(x, w, nullptr, y, c, stream);
        if (rc == -1) rc = f16_generic(x, nullptr, w, y, c, stream);
        return status_of(rc);
    }
    if (!aligned(fws, 16)) return IM2WIN_EINVAL;
    if (fws_bytes < im2win::f16_filter_pack_bytes(c)) return IM2WIN_EWORKSPACE;
    int rc = im2win::launch_f16_filter_pack(w, fws, c, x, stream);
    if (rc == -1) return status_of(f16_generic(x, nullptr, w, y, c, stream));
    if (rc != 0) return status_of(rc);
    rc = im2win::launch_conv_f16_fused(x, w, fws, y, c, stream);
    if (rc == -1) rc = f16_generic(x, nullptr, w, y, c, stream);
    return status_of(rc);
}

// im2col baseline workspace: [padded filter, rounded up to 256 bytes | im2col
// rows of a chunk of images].
struct ColPlan {
    size_t fbytes;     // padded filter bytes (aligned)
    size_t per_image;  // im2col bytes of one image
};

ColPlan col_plan(const ConvShape& c, size_t elem)
{
    const size_t kp = im2win::im2col_row_elems(c, (int)elem);
    return ColPlan{align_up((size_t)c.Co * kp * elem), (size_t)c.Ho * c.Wo * kp * elem};
}

template <typename T>
int im2col_driver(const T* x, const T* w, float* y, void* ws, size_t ws_bytes, int N, int Ci,
                  int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw, hipStream_t stream)
{
    int Ho, Wo;
    if (!x || !w || !y) return IM2WIN_EINVAL;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return IM2WIN_EINVAL;
    if (!aligned(x, sizeof(T)) || !aligned(w, sizeof(T)) || !aligned(y, sizeof(float)))
        return IM2WIN_EINVAL;
    const ConvShape c{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo};
    const ColPlan p = col_plan(c, sizeof(T));
    if (ws == nullptr || ws_bytes < p.fbytes + p.per_image) return IM2WIN_EWORKSPACE;
    if (!aligned(ws, 16)) return IM2WIN_EINVAL;
    unsigned char* wsb = static_cast<unsigned char*>(ws);
    const int64_t x_img = (int64_t)Ci * Hi * Wi, y_img = (int64_t)Co * Ho * Wo;
    // A launch addresses its rows and outputs with 32-bit offsets: below 4 GiB each.
    const size_t lim = 0xFFFFFFF0u;
    size_t cap = std::min<size_t>((size_t)N, (ws_bytes - p.fbytes) / p.per_image);
    cap = std::min(cap, (lim - 1) / p.per_image);
    cap = std::min(cap, (lim - 1) / ((size_t)y_img * 4));
    if (cap < 1) return IM2WIN_EINVAL;
    const int chunk = (int)cap;
    for (int n0 = 0; n0 < N; n0 += chunk) {
        ConvShape cc = c;
        cc.N = std::min(chunk, N - n0);
        int rc = im2win::launch_im2col(x + n0 * x_img, wsb + p.fbytes, cc, (int)sizeof(T), stream);
        if (rc != 0) return status_of(rc);
        rc = im2win::launch_im2col_gemm(wsb + p.fbytes, w, wsb, y + n0 * y_img, cc, (int)sizeof(T),
                                        stream);
        if (rc != 0) return status_of(rc);
    }
    return IM2WIN_OK;
}

template <typename T>
int direct_driver(const T* x, const T* w, float* y, int N, int Ci, int Hi, int Wi, int Co, int Hf,
                  int Wf, int sh, int sw, hipStream_t stream,
                  int (*generic)(const T*, const T*, const T*, float*, const ConvShape&, hipStream_t))
{
    int Ho, Wo;
    if (!x || !w || !y) return IM2WIN_EINVAL;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return IM2WIN_EINVAL;
    if (!aligned(x, sizeof(T)) || !aligned(w, sizeof(T)) || !aligned(y, sizeof(float)))
        return IM2WIN_EINVAL;
    return status_of(generic(x, nullptr, w, y, ConvShape{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo},
                             stream));
}

// NHWC workspace: [filter in the padded window order, rounded up to 256
// bytes | NHWC im2win tensor of a chunk of images, column runs padded to the
// pitch].
ColPlan nhwc_plan(const ConvShape& c, size_t elem)
{
    const size_t pitch = (size_t)im2win::nhwc_pitch(c, (int)elem);
    return ColPlan{align_up((size_t)c.Co * c.Wf * pitch * elem), (size_t)c.Ho * c.Wi * pitch * elem};
}

template <typename T>
int nhwc_driver(const T* x, const T* w, float* y, void* ws, size_t ws_bytes, int N, int Ci, int Hi,
                int Wi, int Co, int Hf, int Wf, int sh, int sw, hipStream_t stream)
{
    int Ho, Wo;
    if (!x || !w || !y) return IM2WIN_EINVAL;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return IM2WIN_EINVAL;
    if (!aligned(x, sizeof(T)) || !aligned(w, sizeof(T)) || !aligned(y, sizeof(float)))
        return IM2WIN_EINVAL;
    const ConvShape c{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo};
    const int e = (int)sizeof(T);
    if (ws == nullptr) {
        if (ws_bytes != 0) return IM2WIN_EWORKSPACE;
        return status_of(im2win::launch_conv_direct_nhwc(x, w, y, c, e, stream));
    }
    const ColPlan p = nhwc_plan(c, sizeof(T));
    if (ws_bytes < p.fbytes + p.per_image) return IM2WIN_EWORKSPACE;
    if (!aligned(ws, 16)) return IM2WIN_EINVAL;
    unsigned char* wsb = static_cast<unsigned char*>(ws);
    int rc = im2win::launch_filter_khwc(w, wsb, c, e, stream);
    if (rc != 0) return status_of(rc);
    const int64_t x_img = (int64_t)Hi * Wi * Ci, y_img = (int64_t)Ho * Wo * Co;
    const size_t lim = 0xFFFFFFF0u;
    size_t cap = std::min<size_t>((size_t)N, (ws_bytes - p.fbytes) / p.per_image);
    cap = std::min(cap, (lim - 1) / p.per_image);
    cap = std::min(cap, (lim - 1) / ((size_t)y_img * 4));
    if (cap < 1) return IM2WIN_EINVAL;
    const int chunk = (int)cap;
    for (int n0 = 0; n0 < N; n0 += chunk) {
        ConvShape cc = c;
        cc.N = std::min(chunk, N - n0);
        rc = im2win::launch_pack_nhwc_padded(x + n0 * x_img, wsb + p.fbytes, cc, e, stream);
        if (rc != 0) return status_of(rc);
        rc = im2win::launch_nhwc_gemm(wsb + p.fbytes, wsb, y + n0 * y_img, cc, e, stream);
        if (rc != 0) return status_of(rc);
    }
    return IM2WIN_OK;
}

}  // namespace

namespace im2win {
int launch_status(hipError_t e)
{
    if (e == hipSuccess) return 0;
    g_last_error = e;
    return -3;
}

void ensure_lds_limit(const void* f, int bytes)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();   // left for the launch to report
        return;
    }
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int> done;
    std::lock_guard<std::mutex> lk(mu);
    int& have = done[std::make_pair(f, dev)];
    if (have >= bytes) return;
    if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
        (void)hipGetLastError();   // the launch reports any limit it exceeds
    else
        have = bytes;
}

const char* const kKnobNames[KNOB_COUNT] = {
    "f32_valu", "f32_nw", "f32_wco", "f32_cb", "f32_ksplit", "f32_occ",
    "f16_rows", "f16_rows_nwv", "f16_rows_bufs", "f16_thin", "f16_thin_nb", "f16_wide",
    "f16_wide_nw", "f16_wpx", "f16_nwh", "tile_order", "f16_reuse", "f16_ws", "sync_staging",
    "f32_small", "f16_res"};

std::atomic<int> g_knobs[KNOB_COUNT];
}  // namespace im2win

extern "C" {

size_t im2win_workspace_bytes_strided(int N, int Ci, int Hi, int Wi, int Hf, int Wf, int sh,
                                      int sw, size_t elem_bytes)
{
    int Ho;
    if (elem_bytes != 2 && elem_bytes != 4) return 0;
    if (!check_shape(N, Ci, Hi, Wi, 1, Hf, Wf, sh, sw, &Ho, nullptr)) return 0;
    return (size_t)N * Ci * Ho * ((size_t)Wi * Hf) * elem_bytes;
}

size_t im2win_workspace_bytes(int N, int Ci, int Hi, int Wi, int Hf, int Wf, int s,
                              size_t elem_bytes)
{
    return im2win_workspace_bytes_strided(N, Ci, Hi, Wi, Hf, Wf, s, s, elem_bytes);
}

int im2win_output_dims_strided(int Hi, int Wi, int Hf, int Wf, int sh, int sw, int* Ho, int* Wo)
{
    return check_shape(1, 1, Hi, Wi, 1, Hf, Wf, sh, sw, Ho, Wo) ? IM2WIN_OK : IM2WIN_EINVAL;
}

int im2win_output_dims(int Hi, int Wi, int Hf, int Wf, int s, int* Ho, int* Wo)
{
    return im2win_output_dims_strided(Hi, Wi, Hf, Wf, s, s, Ho, Wo);
}

int im2win_pack_strided(const void* x, void* ws, int N, int Ci, int Hi, int Wi, int Hf, int Wf,
                        int sh, int sw, size_t elem_bytes, void* stream)
{
    int Ho;
    if (!x || !ws) return IM2WIN_EINVAL;
    if (elem_bytes != 2 && elem_bytes != 4) return IM2WIN_EINVAL;
    if (!check_shape(N, Ci, Hi, Wi, 1, Hf, Wf, sh, sw, &Ho, nullptr)) return IM2WIN_EINVAL;
    if (!aligned(x, elem_bytes) || !aligned(ws, elem_bytes)) return IM2WIN_EINVAL;
    return status_of(im2win::launch_pack(x, ws, N, Ci, Hi, Wi, Hf, sh, Ho, (int)elem_bytes,
                                         static_cast<hipStream_t>(stream)));
}

int im2win_pack(const void* x, void* ws, int N, int Ci, int Hi, int Wi, int Hf, int Wf, int s,
                size_t elem_bytes, void* stream)
{
    return im2win_pack_strided(x, ws, N, Ci, Hi, Wi, Hf, Wf, s, s, elem_bytes, stream);
}

size_t conv2d_im2win_fp16_fused_workspace_bytes(int N, int Ci, int Hi, int Wi, int Co, int Hf,
                                                int Wf, int sh, int sw)
{
    int Ho, Wo;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return 0;
    return align_up(im2win::f16_filter_pack_bytes(ConvShape{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo}));
}

int conv2d_im2win_fp16_fused(const uint16_t* x, const uint16_t* w, float* y, void* fws,
                             size_t fws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf,
                             int Wf, int sh, int sw, void* stream)
{
    return f16_fused_driver(x, w, y, fws, fws_bytes, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw,
                            static_cast<hipStream_t>(stream));
}

int conv2d_im2win_fp32_strided(const float* x, const float* w, float* y, void* ws,
                               size_t ws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf,
                               int Wf, int sh, int sw, void* stream)
{
    return conv_driver<float>(x, w, y, ws, ws_bytes, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw,
                              static_cast<hipStream_t>(stream), f32_fused, f32_from_ws,
                              f32_generic);
}

int conv2d_im2win_fp32(const float* x, const float* w, float* y, void* ws, size_t ws_bytes, int N,
                       int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int s, void* stream)
{
    return conv2d_im2win_fp32_strided(x, w, y, ws, ws_bytes, N, Ci, Hi, Wi, Co, Hf, Wf, s, s,
                                      stream);
}

int conv2d_im2win_fp16_strided(const uint16_t* x, const uint16_t* w, float* y, void* ws,
                               size_t ws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf,
                               int Wf, int sh, int sw, void* stream)
{
    return conv_driver<uint16_t>(x, w, y, ws, ws_bytes, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw,
                                 static_cast<hipStream_t>(stream), im2win::launch_conv_f16_fused,
                                 f16_from_ws, f16_generic);
}

int conv2d_im2win_fp16(const uint16_t* x, const uint16_t* w, float* y, void* ws, size_t ws_bytes,
                       int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int s, void* stream)
{
    return conv2d_im2win_fp16_strided(x, w, y, ws, ws_bytes, N, Ci, Hi, Wi, Co, Hf, Wf, s, s,
                                      stream);
}

size_t conv2d_im2col_workspace_bytes(int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh,
                                     int sw, size_t elem_bytes)
{
    int Ho, Wo;
    if (elem_bytes != 2 && elem_bytes != 4) return 0;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return 0;
    const ColPlan p = col_plan(ConvShape{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo}, elem_bytes);
    return p.fbytes + (size_t)N * p.per_image;
}

int im2col_pack(const void* x, void* col, int N, int Ci, int Hi, int Wi, int Hf, int Wf, int sh,
                int sw, size_t elem_bytes, void* stream)
{
    int Ho, Wo;
    if (!x || !col) return IM2WIN_EINVAL;
    if (elem_bytes != 2 && elem_bytes != 4) return IM2WIN_EINVAL;
    if (!check_shape(N, Ci, Hi, Wi, 1, Hf, Wf, sh, sw, &Ho, &Wo)) return IM2WIN_EINVAL;
    if (!aligned(x, elem_bytes) || !aligned(col, elem_bytes)) return IM2WIN_EINVAL;
    return status_of(im2win::launch_im2col(x, col, ConvShape{N, Ci, Hi, Wi, 1, Hf, Wf, sh, sw, Ho, Wo},
                                           (int)elem_bytes, static_cast<hipStream_t>(stream)));
}

int conv2d_im2col_fp32(const float* x, const float* w, float* y, void* ws, size_t ws_bytes, int N,
                       int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw, void* stream)
{
    return im2col_driver<float>(x, w, y, ws, ws_bytes, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw,
                                static_cast<hipStream_t>(stream));
}

int conv2d_im2col_fp16(const uint16_t* x, const uint16_t* w, float* y, void* ws, size_t ws_bytes,
                       int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw,
                       void* stream)
{
    return im2col_driver<uint16_t>(x, w, y, ws, ws_bytes, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw,
                                   static_cast<hipStream_t>(stream));
}

int conv2d_direct_fp32(const float* x, const float* w, float* y, int N, int Ci, int Hi, int Wi,
                       int Co, int Hf, int Wf, int sh, int sw, void* stream)
{
    return direct_driver<float>(x, w, y, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw,
                                static_cast<hipStream_t>(stream), f32_generic);
}

int conv2d_direct_fp16(const uint16_t* x, const uint16_t* w, float* y, int N, int Ci, int Hi,
                       int Wi, int Co, int Hf, int Wf, int sh, int sw, void* stream)
{
    return direct_driver<uint16_t>(x, w, y, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw,
                                   static_cast<hipStream_t>(stream), f16_generic);
}

size_t conv2d_im2win_nhwc_workspace_bytes(int materialize, int N, int Ci, int Hi, int Wi, int Co,
                                          int Hf, int Wf, int sh, int sw, size_t elem_bytes)
{
    int Ho, Wo;
    if (elem_bytes != 2 && elem_bytes != 4) return 0;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return 0;
    if (!materialize) return 0;
    const ColPlan p = nhwc_plan(ConvShape{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo}, elem_bytes);
    return p.fbytes + (size_t)N * p.per_image;
}

int im2win_pack_nhwc(const void* x, void* ws, int N, int Ci, int Hi, int Wi, int Hf, int Wf, int sh,
                     int sw, size_t elem_bytes, void* stream)
{
    int Ho, Wo;
    if (!x || !ws) return IM2WIN_EINVAL;
    if (elem_bytes != 2 && elem_bytes != 4) return IM2WIN_EINVAL;
    if (!check_shape(N, Ci, Hi, Wi, 1, Hf, Wf, sh, sw, &Ho, &Wo)) return IM2WIN_EINVAL;
    if (!aligned(x, elem_bytes) || !aligned(ws, elem_bytes)) return IM2WIN_EINVAL;
    return status_of(im2win::launch_pack_nhwc(
        x, ws, ConvShape{N, Ci, Hi, Wi, 1, Hf, Wf, sh, sw, Ho, Wo}, (int)elem_bytes,
        static_cast<hipStream_t>(stream)));
}

int conv2d_im2win_nhwc_fp32(const float* x, const float* w, float* y, void* ws, size_t ws_bytes,
                            int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw,
                            void* stream)
{
    return nhwc_driver<float>(x, w, y, ws, ws_bytes, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw,
                              static_cast<hipStream_t>(stream));
}

int conv2d_im2win_nhwc_fp16(const uint16_t* x, const uint16_t* w, float* y, void* ws,
                            size_t ws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf,
                            int sh, int sw, void* stream)
{
    return nhwc_driver<uint16_t>(x, w, y, ws, ws_bytes, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw,
                                 static_cast<hipStream_t>(stream));
}

size_t conv2d_im2win_nhwc_fp16_fused_workspace_bytes(int N, int Ci, int Hi, int Wi, int Co, int Hf,
                                                     int Wf, int sh, int sw)
{
    int Ho, Wo;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return 0;
    return align_up(im2win::f16_interleaved_filter_bytes(ConvShape{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo}));
}

int conv2d_im2win_nhwc_fp16_fused(const uint16_t* x, const uint16_t* w, float* y, void* fws,
                                  size_t fws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf,
                                  int Wf, int sh, int sw, void* stream)
{
    int Ho, Wo;
    if (!x || !w || !y) return IM2WIN_EINVAL;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return IM2WIN_EINVAL;
    if (!aligned(x, 2) || !aligned(w, 2) || !aligned(y, 4)) return IM2WIN_EINVAL;
    const ConvShape c{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo};
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (fws == nullptr) {
        if (fws_bytes != 0) return IM2WIN_EWORKSPACE;
        return status_of(im2win::launch_conv_direct_nhwc(x, w, y, c, 2, st));
    }
    if (fws_bytes < im2win::f16_interleaved_filter_bytes(c)) return IM2WIN_EWORKSPACE;
    if (!aligned(fws, 16)) return IM2WIN_EINVAL;
    if (!im2win::f16_res_applies(c, im2win::kF16CoPad, x, y, true))
        return status_of(im2win::launch_conv_direct_nhwc(x, w, y, c, 2, st));
    int rc = im2win::launch_f16_interleaved_filter_pack(w, fws, c, st);
    if (rc != 0) return status_of(rc);
    return status_of(im2win::launch_conv_f16_res(x, fws, y, c, im2win::kF16CoPad, true, st));
}

const char* im2win_conv_kernel_name(int elem_bytes, int mode, int N, int Ci, int Hi, int Wi,
                                   int Co, int Hf, int Wf, int sh, int sw)
{
    int Ho, Wo;
    if (elem_bytes != 2 && elem_bytes != 4) return nullptr;
    if (mode < 0 || mode > 3 || ((mode == 1 || mode == 3) && elem_bytes != 2)) return nullptr;
    if (!check_shape(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, &Ho, &Wo)) return nullptr;
    const ConvShape c{N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo};
    const void* al = reinterpret_cast<const void*>(uintptr_t(256));
    if (mode == 3)
        return im2win::f16_res_applies(c, im2win::kF16CoPad, al, al, true) ? "conv_f16_res_kernel"
                                                                            : "conv_direct_nhwc_kernel";
    if (elem_bytes == 4) {
        if (mode == 2) return "conv_f32_kernel";
        const char* mfma =
            im2win::knob(im2win::KNOB_F32_VALU) != 1 ? im2win::f32_mfma_kernel_name(c) : nullptr;
        return mfma ? mfma : "conv_f32_kernel";
    }
    if (mode == 2) return im2win::f16_ws_applies(c) ? "conv_f16_ws_kernel" : "conv_f16_kernel";
    return im2win::f16_fused_kernel_name(c, reinterpret_cast<const void*>(uintptr_t(256)), mode == 1);
}

int im2win_set_knob(int knob, int value)
{
    if (knob < 0 || knob >= im2win::KNOB_COUNT) return IM2WIN_EINVAL;
    im2win::g_knobs[knob].store(value, std::memory_order_relaxed);
    return IM2WIN_OK;
}

int im2win_get_knob(int knob)
{
    if (knob < 0 || knob >= im2win::KNOB_COUNT) return 0;
    return im2win::g_knobs[knob].load(std::memory_order_relaxed);
}

const char* im2win_knob_name(int knob)
{
    if (knob < 0 || knob >= im2win::KNOB_COUNT) return nullptr;
    return im2win::kKnobNames[knob];
}

const char* im2win_last_error(void)
{
    return g_last_error == hipSuccess ? "no error" : hipGetErrorString(g_last_error);
}

const char* im2win_status_string(int status)
{
    switch (status) {
    case IM2WIN_OK: return "ok";
    case IM2WIN_EINVAL: return "invalid argument (shape, stride, element size, alignment or NULL pointer)";
    case IM2WIN_EWORKSPACE: return "workspace too small for the requested mode (or size without a buffer)";
    case IM2WIN_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

}  // extern "C"
