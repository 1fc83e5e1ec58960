/*
 * im2win convolution for AMD Instinct MI355X (gfx950): C ABI.
 *
 * The operation is the forward convolution of "Enabling Memory-efficient
 * Im2win Convolution with Multi-precision Support on GPU CUDA and Tensor
 * Cores" (Abstract; Fig. 1; Table I): an NCHW input of N images with Ci
 * channels of Hi x Wi, filters Co x Ci x Hf x Wf, a row stride sh and a
 * column stride sw (Table I writes the stride as s_h(s_w)), and an NCHW
 * output N x Co x Ho x Wo, with
 *     Ho = floor((Hi - Hf) / sh) + 1,   Wo = floor((Wi - Wf) / sw) + 1,
 *     y[n][co][ho][wo] = sum over ci, kh, kw of
 *                        x[n][ci][ho*sh + kh][wo*sw + kw] * w[co][ci][kh][kw]
 * (cross-correlation: no filter flip, no padding, no dilation, no bias; the
 * pages' layers are all unpadded). The same page's Abstract splits the work
 * between general-purpose cores (full precision) and matrix hardware (half
 * precision). Here full precision keeps fp32 inputs, products and sums and
 * runs on the fp32 matrix instructions (a vector-ALU kernel on request);
 * half precision runs on the fp16 matrix instructions with fp32 sums.
 *
 * The im2win transform is the one of "Im2win: Memory Efficient Convolution
 * On SIMD Architectures" (Abstract): each row of dot-product windows is
 * flattened, distinct elements only, into one row. Here the row for
 * (n, ci, ho) holds input rows ho*sh .. ho*sh+Hf-1 over all Wi columns,
 * column by column:
 *     ws[n][ci][ho][w*Hf + kh] = x[n][ci][ho*sh + kh][w]
 * so the window of output (ho, wo) is the single contiguous run of Wf*Hf
 * elements starting at wo*sw*Hf. The workspace is N*Ci*Ho*(Wi*Hf) elements.
 *
 * Each entry point below takes one stride s used for both axes (sh = sw = s,
 * as in every row of Table I); its *_strided twin takes sh and sw and is
 * otherwise identical.
 *
 * Conventions for every entry point:
 *  - Tensors are dense, contiguous, caller-owned DEVICE memory (hipMalloc,
 *    torch). x is N x Ci x Hi x Wi, w is Co x Ci x Hf x Wf, y is
 *    N x Co x Ho x Wo, all row-major. Buffers must not overlap.
 *  - fp16 data is IEEE binary16, passed as uint16_t bit patterns. Outputs of
 *    both convolutions are fp32; the fp16 path multiplies binary16 values
 *    exactly and accumulates in fp32.
 *  - `stream` is a hipStream_t (NULL: the legacy default stream). Work is
 *    enqueued and the call returns without synchronising. The library
 *    allocates no device memory. Its only state is process-wide: the tuning
 *    knobs (im2win_set_knob; default 0 everywhere), per-device kernel
 *    attributes and the fp32 planner's occupancy cache, set up on first use
 *    under a lock. Concurrent calls on different streams are safe when their
 *    output and workspace buffers differ and no knob changes meanwhile.
 *  - Shape limits: every dimension >= 1, Hf <= Hi, Wf <= Wi, strides >= 1, and the
 *    per-image element counts Ci*Hi*Wi, Co*Ho*Wo, Ci*Ho*Wi*Hf and the filter
 *    size Co*Ci*Hf*Wf each below 2^31.
 *  - Argument errors are reported synchronously (no work is enqueued); a
 *    failed kernel launch returns IM2WIN_ELAUNCH. Faults inside a kernel
 *    surface at the caller's next synchronisation, as for any HIP kernel.
 */
#ifndef IM2WIN_H
#define IM2WIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    IM2WIN_OK = 0,
    IM2WIN_EINVAL = -1,     /* bad shape, stride, element size or NULL pointer */
    IM2WIN_EWORKSPACE = -2, /* workspace too small for the mode (or a size with no buffer) */
    IM2WIN_ELAUNCH = -3     /* a kernel launch failed (message: im2win_last_error) */
} im2win_status;

/*
 * Bytes of the im2win tensor for the whole batch:
 *     N * Ci * Ho * (Wi * Hf) * elem_bytes.
 * Returns 0 if the shape is invalid or elem_bytes is not 2 or 4.
 * Pure host arithmetic; needs no GPU.
 */
size_t im2win_workspace_bytes(int N, int Ci, int Hi, int Wi, int Hf, int Wf, int s,
                              size_t elem_bytes);
size_t im2win_workspace_bytes_strided(int N, int Ci, int Hi, int Wi, int Hf, int Wf, int sh,
                                      int sw, size_t elem_bytes);

/*
 * Output extents Ho, Wo (either pointer may be NULL). Returns IM2WIN_OK or
 * IM2WIN_EINVAL. Pure host arithmetic.
 */
int im2win_output_dims(int Hi, int Wi, int Hf, int Wf, int s, int *Ho, int *Wo);
int im2win_output_dims_strided(int Hi, int Wi, int Hf, int Wf, int sh, int sw, int *Ho,
                               int *Wo);

/*
 * The im2win transform (Im2win ... SIMD Architectures, Abstract), as a bit
 * copy of elem_bytes-wide elements (2 or 4; NaN payloads, infinities and
 * subnormals pass unchanged):
 *     ws[n][ci][ho][w*Hf + kh] = x[n][ci][ho*sh + kh][w]
 * x: N x Ci x Hi x Wi; ws: im2win_workspace_bytes(...) bytes, written fully.
 * Wf and sw enter only the shape check (Wo >= 1); the layout of ws does not
 * depend on them. HBM-bound copy kernel.
 */
int im2win_pack(const void *x, void *ws, int N, int Ci, int Hi, int Wi, int Hf, int Wf,
                int s, size_t elem_bytes, void *stream);
int im2win_pack_strided(const void *x, void *ws, int N, int Ci, int Hi, int Wi, int Hf, int Wf,
                        int sh, int sw, size_t elem_bytes, void *stream);

/*
 * fp32 convolution ("full precision" in the GPU page's Abstract): x, w fp32;
 * fp32 products and sums on the fp32 matrix instructions (the vector-ALU
 * kernel with knob "f32_valu" = 1, and for shapes outside the matrix
 * kernel's envelope); y fp32 (written fully).
 *
 * The workspace selects how the im2win rows reach the dot products. With
 * I = one image's im2win bytes (im2win_workspace_bytes with N = 1):
 *  - ws == NULL and ws_bytes == 0: fused. Each workgroup builds the im2win
 *    rows it needs in LDS straight from x; no HBM workspace.
 *  - ws_bytes >= I: materialised (the pages' own formulation). The im2win
 *    tensor of floor(ws_bytes / I) images at a time (at most N; the whole
 *    batch when ws_bytes >= im2win_workspace_bytes(N, ...)) is packed into
 *    the start of the workspace (im2win_pack layout) and convolved from
 *    there, chunk by chunk in stream order. The workspace never needs more
 *    than N * Ci * Ho * Wi * Hf elements.
 *  - anything else (ws == NULL with ws_bytes != 0, or 0 < ws_bytes < I):
 *    IM2WIN_EWORKSPACE; ws not 16-byte aligned: IM2WIN_EINVAL.
 * All modes compute the same windowed dot products; only their fp32
 * summation order may differ. Results of one mode on one shape are the
 * same bits on every call (no atomics, fixed summation order).
 */
int conv2d_im2win_fp32(const float *x, const float *w, float *y, void *ws, size_t ws_bytes,
                       int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int s,
                       void *stream);
int conv2d_im2win_fp32_strided(const float *x, const float *w, float *y, void *ws,
                               size_t ws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf,
                               int Wf, int sh, int sw, void *stream);

/*
 * fp16-input convolution on the matrix cores ("half precision on tensor
 * cores", same Abstract): x, w binary16; products exact, fp32 accumulation;
 * y fp32 (written fully). Workspace rules as for conv2d_im2win_fp32, with
 * elem_bytes = 2; in the fused mode the kernels gather the filter from w.
 */
int conv2d_im2win_fp16(const uint16_t *x, const uint16_t *w, float *y, void *ws,
                       size_t ws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf,
                       int s, void *stream);
int conv2d_im2win_fp16_strided(const uint16_t *x, const uint16_t *w, float *y, void *ws,
                               size_t ws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf,
                               int Wf, int sh, int sw, void *stream);

/*
 * The fused fp16 convolution with its filter staging split out: the filter is
 * first re-laid out ("prepacked") into fws in the order of the K slices of
 * the matrix-core kernel the shape runs on, then that kernel copies its
 * slices straight from fws instead of gathering them from w. Same results as
 * conv2d_im2win_fp16 without a workspace (same kernel, same summation order).
 * Strides per axis, as the *_strided calls.
 *  - conv2d_im2win_fp16_fused_workspace_bytes: bytes fws needs for the shape
 *    (a multiple of 256; depends on the shape only); 0 for an invalid shape.
 *  - conv2d_im2win_fp16_fused: fws (16-byte aligned, caller-owned, at least
 *    that many bytes, overwritten) holds the prepacked filter during the
 *    call; fws == NULL with fws_bytes == 0 gathers the filter in the kernel.
 *    A smaller fws, or a size without a buffer: IM2WIN_EWORKSPACE.
 */
size_t conv2d_im2win_fp16_fused_workspace_bytes(int N, int Ci, int Hi, int Wi, int Co, int Hf,
                                                int Wf, int sh, int sw);
int conv2d_im2win_fp16_fused(const uint16_t *x, const uint16_t *w, float *y, void *fws,
                             size_t fws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf,
                             int Wf, int sh, int sw, void *stream);

/*
 * conv2d_im2win_fp16_fused for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the prepacked filter goes to a fixed 4 MiB array in each
 * device's global memory that the library holds until the process ends,
 * instead of a caller workspace. The call itself allocates nothing. Same
 * results as conv2d_im2win_fp16_fused (same kernels). A shape whose
 * conv2d_im2win_fp16_fused_workspace_bytes exceeds 4 MiB (4194304) returns
 * IM2WIN_EWORKSPACE before anything is enqueued; an invalid shape or pointer
 * IM2WIN_EINVAL. Every call on one device uses that device's array: calls
 * that overlap on one device (other streams or threads) race and must be
 * serialised by the caller.
 */
int conv2d_im2win_fp16_fused_noalloc(const uint16_t *x, const uint16_t *w, float *y, int N,
                                     int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw,
                                     void *stream);

/*
 * Baselines the pages compare im2win against, built here on the same
 * hardware paths (they carry the row and column strides directly):
 *
 * im2col + GEMM ("Enabling Memory-efficient Im2win Convolution ...", Fig. 1
 * right; Abstract: GEMM-based convolution). The im2col matrix holds, for every
 * output pixel q = (n*Ho + ho)*Wo + wo, its receptive field as one row of
 * K = Ci*Hf*Wf elements in (ci, kh, kw) order, zero-padded to KP elements
 * (K rounded up to 32 bytes):
 *     col[q][(ci*Hf + kh)*Wf + kw] = x[n][ci][ho*sh + kh][wo*sw + kw]
 * (the transpose of the K x P layout, same size). im2col_pack writes it for N
 * images (N*Ho*Wo*KP elements; elem_bytes 2 or 4, bit copy).
 * conv2d_im2col_workspace_bytes: bytes for the whole batch, laid out as
 * [filter padded to KP per channel, rounded up to 256 bytes | im2col rows].
 * conv2d_im2col_fp32 / _fp16: the convolution as im2col then a matrix-core
 * GEMM (same MFMA instructions and accumulation as the im2win kernels); ws
 * is required (16-byte aligned) and must hold the padded filter and at least
 * one image's rows; the batch is processed in chunks of as many images as
 * fit. Smaller: IM2WIN_EWORKSPACE. Results as conv2d_im2win_fp32 / _fp16
 * (fp32 output; only the summation order differs).
 *
 * conv2d_direct_fp32 / _fp16: direct convolution, one thread per output,
 * reading x and w in place (no workspace).
 */
size_t conv2d_im2col_workspace_bytes(int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh,
                                     int sw, size_t elem_bytes);
int im2col_pack(const void *x, void *col, int N, int Ci, int Hi, int Wi, int Hf, int Wf, int sh,
                int sw, size_t elem_bytes, void *stream);
int conv2d_im2col_fp32(const float *x, const float *w, float *y, void *ws, size_t ws_bytes, int N,
                       int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw, void *stream);
int conv2d_im2col_fp16(const uint16_t *x, const uint16_t *w, float *y, void *ws, size_t ws_bytes,
                       int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw,
                       void *stream);
int conv2d_direct_fp32(const float *x, const float *w, float *y, int N, int Ci, int Hi, int Wi,
                       int Co, int Hf, int Wf, int sh, int sw, void *stream);
int conv2d_direct_fp16(const uint16_t *x, const uint16_t *w, float *y, int N, int Ci, int Hi,
                       int Wi, int Co, int Hf, int Wf, int sh, int sw, void *stream);

/*
 * NHWC tensors: x is N x Hi x Wi x Ci, y is N x Ho x Wo x Co (fp32), w stays
 * Co x Ci x Hf x Wf. The im2win transform keeps the channels innermost
 * (the flattening of "Im2win: Memory Efficient Convolution On SIMD
 * Architectures", Abstract, in this layout):
 *     ws[n][ho][w][kh][c] = x[n][ho*sh + kh][w][c]
 * so the window of output (ho, wo) is the one contiguous run of Wf*Hf*Ci
 * elements at wo*sw*Hf*Ci in row (n, ho). Same size as the NCHW tensor
 * (im2win_workspace_bytes_strided).
 *
 * im2win_pack_nhwc: that transform (bit copy, elem_bytes 2 or 4).
 * conv2d_im2win_nhwc_workspace_bytes: 0 without materialize; with it, the
 *     bytes of [filter in window order, rounded up to 256 | the NHWC im2win
 *     tensor of the whole batch], where each column's run of Hf*Ci elements
 *     is stored in pitch = Hf*Ci rounded up to 32 bytes (16 halves, 8
 *     floats), zeros after it, and each filter row holds Wf such runs:
 *         ws[((n*Ho + ho)*Wi + w)*pitch + kh*Ci + c] = x[n][ho*sh + kh][w][c]
 *         wr[co*Wf*pitch + kw*pitch + kh*Ci + c]    = w[co][c][kh][kw]
 *     (pitch == Hf*Ci, the tensor above unchanged, when Ci*elem_bytes is a
 *     multiple of 32).
 * conv2d_im2win_nhwc_fp32 / _fp16: ws == NULL and ws_bytes == 0: direct
 *     convolution (one thread per output). ws (16-byte aligned) with at least
 *     the filter part and one image's tensor: materialised; the tensor of as
 *     many images as fit is packed and multiplied on the matrix cores, the
 *     padded window runs as GEMM rows, for every shape. A workspace given
 *     but too small: IM2WIN_EWORKSPACE.
 */
size_t conv2d_im2win_nhwc_workspace_bytes(int materialize, int N, int Ci, int Hi, int Wi, int Co,
                                          int Hf, int Wf, int sh, int sw, size_t elem_bytes);
int im2win_pack_nhwc(const void *x, void *ws, int N, int Ci, int Hi, int Wi, int Hf, int Wf,
                     int sh, int sw, size_t elem_bytes, void *stream);
int conv2d_im2win_nhwc_fp32(const float *x, const float *w, float *y, void *ws, size_t ws_bytes,
                            int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf, int sh, int sw,
                            void *stream);
int conv2d_im2win_nhwc_fp16(const uint16_t *x, const uint16_t *w, float *y, void *ws,
                            size_t ws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf, int Wf,
                            int sh, int sw, void *stream);

/*
 * The fused fp16 NHWC convolution (the half-precision path of "Enabling
 * Memory-efficient Im2win Convolution with Multi-precision Support on GPU
 * CUDA and Tensor Cores", Abstract, on NHWC tensors): no im2win tensor in
 * HBM. In NHWC the 8 channels of one input pixel are 16 contiguous bytes,
 * so a tile's input rows are copied into LDS as they lie; each workgroup
 * keeps them there and multiplies them with the filter, prepacked into fws,
 * on the matrix cores. x is N x Hi x Wi x Ci (fp16), y N x Ho x Wo x Co
 * (fp32), w Co x Ci x Hf x Wf (fp16).
 *
 * conv2d_im2win_nhwc_fp16_fused_workspace_bytes: the bytes of the prepacked
 *     filter (16-byte entries of 8 input channels of one tap for one output
 *     channel); 0 for an invalid shape.
 * conv2d_im2win_nhwc_fp16_fused: fws (16-byte aligned) with at least that
 *     many bytes: the filter is packed into it, then the resident-input
 *     kernel runs when the shape is in its envelope (Co a multiple of 256,
 *     Ci of 8, at least 4 taps, x and y 16-byte aligned, a tile's input rows
 *     within LDS; im2win_conv_kernel_name mode 3 names the kernel); other
 *     shapes, and fws == NULL with fws_bytes == 0, take the direct NHWC
 *     kernel. fws given but too small: IM2WIN_EWORKSPACE; fws not 16-byte
 *     aligned: IM2WIN_EINVAL. The caller owns every buffer; fws holds the
 *     packed filter afterwards.
 */
size_t conv2d_im2win_nhwc_fp16_fused_workspace_bytes(int N, int Ci, int Hi, int Wi, int Co,
                                                     int Hf, int Wf, int sh, int sw);
int conv2d_im2win_nhwc_fp16_fused(const uint16_t *x, const uint16_t *w, float *y, void *fws,
                                  size_t fws_bytes, int N, int Ci, int Hi, int Wi, int Co, int Hf,
                                  int Wf, int sh, int sw, void *stream);

/*
 * Tuning knobs of the kernel planners, for tests and the ablation study
 * (the pages' variant study, Table II and Fig. 4 of "Enabling
 * Memory-efficient Im2win Convolution ..."). Knob k is named by
 * im2win_knob_name(k) (NULL past the last one); every knob is 0 by default,
 * meaning the planner's choice. A knob selects which kernel, tiling, tile
 * order or staging runs; it never changes a workspace size or any result
 * beyond the fp32 summation order. Process-wide; set them only while no call
 * runs. im2win_set_knob returns IM2WIN_OK, or IM2WIN_EINVAL for an unknown
 * knob; im2win_get_knob returns the value (0 for an unknown knob).
 */
int im2win_set_knob(int knob, int value);
int im2win_get_knob(int knob);
const char *im2win_knob_name(int knob);

/*
 * Name of the main kernel a convolution call with this shape runs under the
 * current knobs (for profiles and reports), assuming x 16-byte aligned.
 * elem_bytes 4 (conv2d_im2win_fp32) or 2 (the fp16 calls); mode 0: fused (no
 * workspace), 1: conv2d_im2win_fp16_fused with a filter workspace, 2:
 * materialised (the im2win_pack launches come first), 3:
 * conv2d_im2win_nhwc_fp16_fused with a filter workspace (fp16 only; y also
 * 16-byte aligned). Static string; NULL for an invalid shape or mode. Host
 * only.
 */
const char *im2win_conv_kernel_name(int elem_bytes, int mode, int N, int Ci, int Hi, int Wi,
                                   int Co, int Hf, int Wf, int sh, int sw);

/*
 * Rate probe (a measurement helper, not part of the convolution): enqueues
 * `blocks` workgroups of 4 waves, each running `iters` rounds of arithmetic
 * on registers only, and writes one float per thread into out (device
 * memory, blocks * 256 floats, caller-owned; the values are meaningless).
 * kind 0: fp32 vector FMA (unpacked, 8 chains per lane), 1: fp32 matrix
 * instruction v_mfma_f32_32x32x2_f32, 2: fp16 matrix instruction
 * v_mfma_f32_32x32x16_f16 (4 independent accumulators per wave). Timed by
 * the caller, it gives the rate the chip sustains for that kind of work
 * (the measured peak beside the published one). im2win_peak_probe_flops
 * returns the flops one launch performs (0 for invalid arguments).
 * Returns IM2WIN_OK, IM2WIN_EINVAL or IM2WIN_ELAUNCH.
 */
int im2win_peak_probe(int kind, int blocks, int iters, float *out, void *stream);
double im2win_peak_probe_flops(int kind, int blocks, int iters);

/* Static, human-readable text for a status code. */
const char *im2win_status_string(int status);

/*
 * Text of the HIP runtime error behind the last IM2WIN_ELAUNCH returned on
 * the calling thread ("no error" if there was none). Static storage.
 */
const char *im2win_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IM2WIN_H */
