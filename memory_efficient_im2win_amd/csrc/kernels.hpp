// Kernel launchers shared by the C-ABI layer. Each returns 0 on success,
// -1 if the shape is outside what the launcher supports, -3 if the launch
// failed. Shapes are validated by the caller first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace im2win {

// Result of the launches just enqueued: 0 if the runtime reports no error,
// else -3, keeping the error for im2win_last_error() on this thread.
int launch_status(hipError_t e);
inline int launch_status() { return launch_status(hipGetLastError()); }

// Convolution geometry of one launch (N = images in this launch); sh and sw
// are the row and column strides.
struct ConvShape {
    int N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, Ho, Wo;
};

// The im2win transform of N images (bit copy of elem_bytes-wide elements).
// Only the row stride sh enters it.
int launch_pack(const void* x, void* ws, int N, int Ci, int Hi, int Wi, int Hf, int sh, int Ho,
                int elem_bytes, hipStream_t stream);

// fp32 convolution on the vector ALUs. ws == nullptr: im2win rows are built
// in LDS from x; otherwise they are read from the packed tensor ws (N images).
int launch_conv_f32(const float* x, const float* ws, const float* w, float* y,
                    const ConvShape& c, hipStream_t stream);

// fp32 convolution on the matrix cores (v_mfma_f32_32x32x2_f32), window
// tiles built in LDS from x. -1 if the shape is outside its envelope. Small
// problems split K over the waves of a workgroup (fixed-order sums).
int launch_conv_f32_mfma(const float* x, const float* w, float* y, const ConvShape& c,
                         hipStream_t stream);
bool f32_mfma_applies(const ConvShape& c);
// The fp32 matrix-core kernel the planner runs for shape c:
// "conv_f32_mfma_kernel" or "conv_f32_small_kernel" (nullptr: neither).
const char* f32_mfma_kernel_name(const ConvShape& c);

// fp32 convolution for problems whose output tiles cannot fill the chip
// (v_mfma_f32_16x16x4_f32, one stage, K split over a workgroup's waves);
// -1 if the shape is outside its envelope.
bool f32_small_applies(const ConvShape& c);
int launch_conv_f32_small(const float* x, const float* w, float* y, const ConvShape& c,
                          hipStream_t stream);

// fp16 convolution from the materialised tensor ws (N images) with each
// channel's window stretch copied into LDS by direct loads (f16_ws_applies);
// -1 if the shape or ws's alignment is outside its envelope.
bool f16_ws_applies(const ConvShape& c);
int launch_conv_f16_ws(const uint16_t* ws, const uint16_t* w, float* y, const ConvShape& c,
                       hipStream_t stream);

// fp16 x fp16 -> fp32 convolution on the matrix cores; ws as above.
int launch_conv_f16(const uint16_t* x, const uint16_t* ws, const uint16_t* w, float* y,
                    const ConvShape& c, hipStream_t stream);

// Fused fp16 convolution (im2win window tiles built in LDS). wpk is the
// filter prepacked by launch_f16_filter_pack for the same shape and x, or
// nullptr to gather the filters from w inside the kernel. -1 if the shape is
// outside every tiled kernel's envelope.
int launch_conv_f16_fused(const uint16_t* x, const uint16_t* w, const void* wpk, float* y,
                          const ConvShape& c, hipStream_t stream);
// Bytes that hold the prepacked fp16 filter in the layout of any fused
// kernel (depends on the shape only). The pack writes the layout of the
// kernel the call with this shape and x runs on (-1: none of them takes it).
size_t f16_filter_pack_bytes(const ConvShape& c);
int launch_f16_filter_pack(const uint16_t* w, void* wpk, const ConvShape& c, const void* x,
                           hipStream_t stream);
// Name of the kernel launch_conv_f16_fused runs for this shape and x.
const char* f16_fused_kernel_name(const ConvShape& c, const void* x, bool prepacked);

// Raises kernel f's dynamic LDS limit to `bytes` on the current device, once
// per (kernel, device); thread-safe. A failure is left for the launch to
// report.
void ensure_lds_limit(const void* f, int bytes);

// fp16 convolution with the input rows copied to LDS by direct loads and the
// filter prepacked by launch_f16_rows_filter_pack (its own layout; wp), or
// gathered from w when wp is nullptr. Used by the three calls above for the
// shapes it takes (f16_rows_applies). -1 if the shape or x's alignment is
// outside its envelope.
bool f16_rows_applies(const ConvShape& c);
size_t f16_rows_filter_bytes(const ConvShape& c);
int launch_f16_rows_filter_pack(const uint16_t* w, void* wp, const ConvShape& c,
                                hipStream_t stream);
int launch_conv_f16_rows(const uint16_t* x, const void* wp, const uint16_t* w, float* y,
                         const ConvShape& c, hipStream_t stream);
// The same filter layout, slices (c, kh) of the 8 taps kw, channels padded
// to a multiple of 64, for any shape with Wf <= 8 and Hf*Wf <= 256.
size_t f16_slices_filter_bytes(const ConvShape& c);
int launch_f16_slices_filter_pack(const uint16_t* w, void* wp, const ConvShape& c,
                                  hipStream_t stream);

// fp16 convolution of the row-staged kernel's shapes (its filter layout)
// with each staged input row reused across the output rows that share it
// and the filter held in registers (f16_reuse_applies). -1 if the shape or
// x's alignment is outside its envelope.
bool f16_reuse_applies(const ConvShape& c);
int launch_conv_f16_reuse(const uint16_t* x, const void* wp, const uint16_t* w, float* y,
                          const ConvShape& c, hipStream_t stream);

// fp16 convolution for thin layers (few input channels: the whole filter
// stays in LDS as slices (c, kh) of 8 taps), reading the filter packed by
// launch_f16_slices_filter_pack (wp), or gathering it from w when wp is
// nullptr. Used by launch_conv_f16_fused for the shapes it takes
// (f16_thin_applies) that the row-staged kernel does not.
bool f16_thin_applies(const ConvShape& c);
int launch_conv_f16_thin(const uint16_t* x, const void* wp, const uint16_t* w, float* y,
                         const ConvShape& c, hipStream_t stream);

// fp16 convolution for layers with many output channels (128-channel wave
// tiles), reading the filter prepacked by launch_f16_filter_pack with its
// channels padded to a multiple of copad_mult (wpk), or gathering it from w
// when wpk is nullptr. Used by launch_conv_f16_fused for the shapes it takes
// (f16_wide_applies) that the row-staged and thin-layer kernels do not.
bool f16_wide_applies(const ConvShape& c, size_t copad_mult);
int launch_conv_f16_wide(const uint16_t* x, const void* wpk, const uint16_t* w, float* y,
                         const ConvShape& c, size_t copad_mult, hipStream_t stream);

// fp16 convolution with a tile's input rows resident in LDS and the filter,
// prepacked as for the wide-tile kernel (channels padded to a multiple of
// copad_mult), read into registers: 256 output channels x whole output rows
// of one image per workgroup. Used by launch_conv_f16_fused for prepacked
// calls on the shapes it takes (f16_res_applies) that
// would otherwise run on the wide-tile or channel-interleaved kernel (x and
// y 16-byte aligned). nhwc: x is N x Hi x Wi x Ci and y N x Ho x Wo x Co
// (the fused NHWC call).
bool f16_res_applies(const ConvShape& c, size_t copad_mult, const void* x, const void* y,
                     bool nhwc = false);
int launch_conv_f16_res(const uint16_t* x, const void* wpk, float* y, const ConvShape& c,
                        size_t copad_mult, bool nhwc, hipStream_t stream);
// The channel-interleaved filter entries of the wide-tile and resident-input
// kernels, [(g*HWp + j)*Copad + co] = w[co][8g..8g+7][j], whatever kernel the
// NCHW planner would pick for the shape.
int launch_f16_interleaved_filter_pack(const uint16_t* w, void* wpk, const ConvShape& c,
                                       hipStream_t stream);
// Output channels of those entries are padded to a multiple of this; their
// bytes: ceil(Ci/8) x HWp x Copad x 16.
constexpr int kF16CoPad = 128;
size_t f16_interleaved_filter_bytes(const ConvShape& c);

// im2col + GEMM baseline: elements per im2col row (Ci*Hf*Wf padded to 32
// bytes); the transform of N images into N*Ho*Wo rows; the GEMM over those
// rows, after copying the filters into wpad (Co rows of the padded length).
size_t im2col_row_elems(const ConvShape& c, int elem);
int launch_im2col(const void* x, void* col, const ConvShape& c, int elem, hipStream_t stream);
int launch_im2col_gemm(const void* col, const void* w, void* wpad, float* y, const ConvShape& c,
                       int elem, hipStream_t stream);

// NHWC (x: N x Hi x Wi x Ci, y: N x Ho x Wo x Co): the im2win transform
// ws[n][ho][w][kh][c] = x[n][ho*sh + kh][w][c] (unpadded, and with each
// column's Hf*Ci run padded with zeros to nhwc_pitch elements, a multiple of
// 32 bytes); the filters reordered to the padded window order
// wr[co][kw*pitch + kh*Ci + c]; the GEMM over the padded window runs; the
// direct kernel.
int nhwc_pitch(const ConvShape& c, int elem);
int launch_pack_nhwc(const void* x, void* ws, const ConvShape& c, int elem, hipStream_t stream);
int launch_pack_nhwc_padded(const void* x, void* ws, const ConvShape& c, int elem,
                            hipStream_t stream);
int launch_filter_khwc(const void* w, void* wr, const ConvShape& c, int elem, hipStream_t stream);
int launch_nhwc_gemm(const void* ws, const void* wr, float* y, const ConvShape& c, int elem,
                     hipStream_t stream);
int launch_conv_direct_nhwc(const void* x, const void* w, float* y, const ConvShape& c, int elem,
                            hipStream_t stream);

// Plain fallbacks (one thread per output) for shapes the tiled kernels do
// not take; ws as above.
int launch_conv_generic_f32(const float* x, const float* ws, const float* w, float* y,
                            const ConvShape& c, hipStream_t stream);
int launch_conv_generic_f16(const uint16_t* x, const uint16_t* ws, const uint16_t* w, float* y,
                            const ConvShape& c, hipStream_t stream);

}  // namespace im2win
