/*
 * miconv.h -- C ABI of libmiconv, the 2-D convolution forward pass (FPROP)
 * its data and filter gradients, and pooling, for AMD Instinct MI355X (gfx950).
 *
 * The operation (direct convolution, cross-correlation form, zero padding):
 *
 *   y[n,k,p,q] = alpha * sum_{c,r,s} X(n, c, p*u + r - pad_top, q*v + s - pad_left) * F[k,c,r,s]
 *              + beta  * y[n,k,p,q]
 *
 *   X(n,c,h,w) = x[n*sn + c*sc + h*sh + w*sw] inside 0 <= h < H, 0 <= w < W, else 0
 *   P = floor((H + pad_top + pad_bottom - R) / u) + 1
 *   Q = floor((W + pad_left + pad_right - S) / v) + 1
 *
 * Sources: cuDNN page (Chetlur et al., "cuDNN: Efficient Primitives for Deep
 * Learning"), "Proposed Method": a C API over opaque tensor and filter
 * descriptors with arbitrary strides and layouts, single and double
 * precision, user-owned GPU memory and no auxiliary buffers, non-square
 * inputs and asymmetric padding.  maxDNN page (Lavin), "Proposed Method":
 * each output coordinate is the product of the input receptive field with
 * the filter weights.  Zero-memory direct-convolution page (Zhang, Franchetti
 * et al.), Abstract and "Proposed Method": computed directly, without packing
 * or copying, with no memory beyond the operands.
 *
 * Conventions for every call:
 *   - Every call returns a mic_status; nothing is thrown across the ABI.
 *   - Descriptors and handles are host objects owned by the caller (create /
 *     destroy).  They hold no device memory.
 *   - Data pointers are device pointers owned by the caller.  The library
 *     never allocates, frees or keeps device memory: there is no workspace.
 *   - Strides are counted in elements, not bytes, and must be >= 1.
 *   - Not thread-safe per handle: one handle, one host thread at a time.
 */
#ifndef MICONV_H
#define MICONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MICONV_VERSION_MAJOR 0
#define MICONV_VERSION_MINOR 1
#define MICONV_VERSION_PATCH 0

typedef enum {
    MIC_STATUS_SUCCESS = 0,
    MIC_STATUS_BAD_PARAM = 1,       /* null pointer, bad dimension/stride, shape mismatch */
    MIC_STATUS_NOT_SUPPORTED = 2,   /* valid request this library does not implement */
    MIC_STATUS_LAUNCH_FAILED = 3,   /* the HIP runtime refused a kernel launch */
    MIC_STATUS_INTERNAL_ERROR = 4,  /* HIP runtime error outside a launch (device query) */
    MIC_STATUS_ALLOC_FAILED = 5     /* host allocation of a handle or descriptor failed */
} mic_status;

/* Element types.  Allowed (x, w, y) combinations: (F32, F32, F32),
 * (F64, F64, F64) and (BF16, BF16, F32) (bf16 inputs, fp32 accumulation and
 * output).  Anything else is MIC_STATUS_NOT_SUPPORTED. */
typedef enum {
    MIC_DTYPE_F32 = 0,
    MIC_DTYPE_F64 = 1,
    MIC_DTYPE_BF16 = 2
} mic_dtype;

/* Packed layouts for mic_tensor_desc_set_packed.  Any other layout is given
 * through explicit strides with mic_tensor_desc_set. */
typedef enum {
    MIC_LAYOUT_NCHW = 0,
    MIC_LAYOUT_NHWC = 1
} mic_layout;

typedef struct mic_handle_st* mic_handle;
typedef struct mic_tensor_desc_st* mic_tensor_desc;
typedef struct mic_filter_desc_st* mic_filter_desc;
typedef struct mic_conv_desc_st* mic_conv_desc;

/* Static, never-NULL text for a status (unknown values give "unknown status"). */
const char* mic_status_string(mic_status status);

/* Library version; any pointer may be NULL. */
mic_status mic_get_version(int* major, int* minor, int* patch);

/* ---------------------------------------------------------------- handle */

/* Binds the calling thread's current HIP device and the null stream.
 * Queries the device (compute-unit count, architecture); fails with
 * MIC_STATUS_INTERNAL_ERROR when no HIP device is usable and with
 * MIC_STATUS_NOT_SUPPORTED on a device other than gfx950.  No device memory
 * is allocated. */
mic_status mic_create(mic_handle* handle);
mic_status mic_destroy(mic_handle handle);

/* stream is a hipStream_t (NULL = the null stream).  Later calls on this
 * handle enqueue their kernels on it.  The caller keeps the stream alive. */
mic_status mic_set_stream(mic_handle handle, void* stream);
mic_status mic_get_stream(mic_handle handle, void** stream);

/* ---------------------------------------------------------------- tensor descriptor */

mic_status mic_tensor_desc_create(mic_tensor_desc* desc);
mic_status mic_tensor_desc_destroy(mic_tensor_desc desc);

/* Logical N, C, H, W with element strides sn, sc, sh, sw (any order, any
 * gaps: NCHW, NHWC, padded rows and sub-tensor views all fit).  Dimensions
 * and strides must be >= 1, else MIC_STATUS_BAD_PARAM. */
mic_status mic_tensor_desc_set(mic_tensor_desc desc, mic_dtype dtype,
                               int n, int c, int h, int w,
                               int64_t sn, int64_t sc, int64_t sh, int64_t sw);

/* Same, with the strides of a packed NCHW or NHWC tensor. */
mic_status mic_tensor_desc_set_packed(mic_tensor_desc desc, mic_dtype dtype, mic_layout layout,
                                      int n, int c, int h, int w);

/* Read back; any output pointer may be NULL.  strides receives 4 values
 * (sn, sc, sh, sw).  MIC_STATUS_BAD_PARAM if the descriptor was never set. */
mic_status mic_tensor_desc_get(mic_tensor_desc desc, mic_dtype* dtype,
                               int* n, int* c, int* h, int* w, int64_t* strides);

/* Channel-blocked tensor (zero-memory direct-convolution page, "Proposed
 * Method": input and output feature maps in a blocked layout that takes
 * exactly the memory of standard storage): packed [N][C/cb][H][W][cb], so
 * element (n, c, h, w) sits at
 *   n*C*H*W + (c / cb)*H*W*cb + h*W*cb + w*cb + (c % cb).
 * c must be a multiple of cb (no padding channels), cb >= 1, else
 * MIC_STATUS_BAD_PARAM.  Accepted by mic_conv_forward for x and y, any cb:
 * the tap-batched kernels read blocked x when cb is a multiple of their
 * channel chunk (2 or 4 channels fp32/fp64, 16 bf16), the row-streamed
 * kernel (11-wide filter rows) when it is a multiple of 4 and x is 16-byte
 * aligned, the gather kernel's tap order when it is a multiple of 16 (32
 * bf16); other blockings run the gather kernel's flat order or the direct
 * kernel.  The other operations
 * return MIC_STATUS_NOT_SUPPORTED for blocked descriptors.
 * mic_tensor_desc_set / _set_packed reset a descriptor to unblocked. */
mic_status mic_tensor_desc_set_blocked(mic_tensor_desc desc, mic_dtype dtype, int n, int c, int h, int w,
                                       int cb);

/* Channel block cb (0 for an unblocked descriptor) and the element stride
 * between channel blocks; either pointer may be null.  MIC_STATUS_BAD_PARAM
 * if the descriptor was never set. */
mic_status mic_tensor_desc_get_block(mic_tensor_desc desc, int* cb, int64_t* block_stride);

/* ---------------------------------------------------------------- filter descriptor */

mic_status mic_filter_desc_create(mic_filter_desc* desc);
mic_status mic_filter_desc_destroy(mic_filter_desc desc);

/* K filters of C channels and R x S taps, packed K,C,R,S (S fastest).
 * Dimensions must be >= 1. */
mic_status mic_filter_desc_set(mic_filter_desc desc, mic_dtype dtype, int k, int c, int r, int s);
mic_status mic_filter_desc_get(mic_filter_desc desc, mic_dtype* dtype, int* k, int* c, int* r, int* s);

/* Blocked filters (zero-memory direct-convolution page, "Proposed Method":
 * kernel weights in a blocked layout of the same size as standard storage):
 * [K/kb][C/cb][R][S][cb][kb], so F[k, c, r, s] sits at
 *   ((k/kb)*(C/cb) + c/cb)*R*S*cb*kb + ((r*S + s)*cb + c%cb)*kb + k%kb.
 * k must be a multiple of kb and c of cb (kb, cb >= 1), else
 * MIC_STATUS_BAD_PARAM.  Forward pass only, as for blocked tensors: the
 * tap-batched kernels read them when cb is a multiple of their channel
 * chunk and kb of 4 (fp32), 2 (fp64) or 8 (bf16, cb a multiple of 16) with
 * w 16-byte aligned, the row-streamed kernel tap by tap, the gather kernel
 * when cb is a multiple of 16 (32 bf16), else the direct kernel runs.
 * mic_filter_desc_set resets a descriptor to packed KCRS. */
mic_status mic_filter_desc_set_blocked(mic_filter_desc desc, mic_dtype dtype, int k, int c, int r, int s,
                                       int kb, int cb);

/* Filter blocks kb, cb (0, 0 for packed KCRS); either pointer may be null.
 * MIC_STATUS_BAD_PARAM if the descriptor was never set. */
mic_status mic_filter_desc_get_block(mic_filter_desc desc, int* kb, int* cb);

/* ---------------------------------------------------------------- convolution descriptor */

mic_status mic_conv_desc_create(mic_conv_desc* desc);
mic_status mic_conv_desc_destroy(mic_conv_desc desc);

/* Per-side zero padding (>= 0) and stride u along H, v along W (>= 1).
 * No dilation, no groups, no filter flip. */
mic_status mic_conv_desc_set(mic_conv_desc desc, int pad_top, int pad_bottom,
                             int pad_left, int pad_right, int stride_h, int stride_w);
mic_status mic_conv_desc_get(mic_conv_desc desc, int* pad_top, int* pad_bottom,
                             int* pad_left, int* pad_right, int* stride_h, int* stride_w);

/* ---------------------------------------------------------------- forward */

/* Output dimensions (N, K, P, Q).  Host only, no device needed.
 * MIC_STATUS_BAD_PARAM if a descriptor is unset, the channel counts differ,
 * or the output would be empty (P < 1 or Q < 1). */
mic_status mic_conv_forward_output_dim(mic_conv_desc conv, mic_tensor_desc x_desc,
                                       mic_filter_desc w_desc, int* n, int* k, int* p, int* q);

/* y <- alpha * conv(x, w) + beta * y, on the handle's stream, asynchronously.
 *
 * x: device memory described by x_desc; w: packed K,C,R,S device memory;
 * y: device memory described by y_desc, whose dims must equal the output
 * dims.  alpha and beta are rounded to the accumulation type (fp32 for F32
 * and BF16 inputs, fp64 for F64).  With beta == 0, y is only written (its
 * old contents, NaN included, never reach the result).
 *
 * No workspace: nothing is allocated.  The return value covers validation
 * and the launch only; execution errors surface at the next synchronisation.
 * y must not overlap x or w, and y's strides must not map two outputs to one
 * address (neither is checked).  Tensors whose highest element offset
 * reaches 2^31 are MIC_STATUS_NOT_SUPPORTED.
 *
 * Errors: MIC_STATUS_BAD_PARAM (null handle/descriptor/pointer, unset
 * descriptor, shape mismatch), MIC_STATUS_NOT_SUPPORTED (dtype combination,
 * size limit), MIC_STATUS_LAUNCH_FAILED. */
mic_status mic_conv_forward(mic_handle handle, double alpha,
                            mic_tensor_desc x_desc, const void* x,
                            mic_filter_desc w_desc, const void* w,
                            mic_conv_desc conv, double beta,
                            mic_tensor_desc y_desc, void* y);

/* Name of the kernel variant mic_conv_forward would launch for these
 * descriptors (host only; for profiling and reports).  Writes a NUL-
 * terminated string of at most buflen bytes; MIC_STATUS_BAD_PARAM if the
 * descriptors are invalid or buflen is too small. */
mic_status mic_conv_forward_kernel_name(mic_handle handle, mic_tensor_desc x_desc,
                                        mic_filter_desc w_desc, mic_conv_desc conv,
                                        mic_tensor_desc y_desc, char* buf, size_t buflen);

/* ---------------------------------------------------------------- data gradient */

/* dx <- alpha * dgrad(dy, w) + beta * dx: the backward pass with respect to
 * the input, i.e. the adjoint of the forward sum in x,
 *
 *   dx[n,c,h,w] = alpha * sum_{k,r,s} dY(n, k, p, q) * F[k,c,r,s]
 *                 over p*u = h + pad_top - r (0 <= p < P),
 *                      q*v = w + pad_left - s (0 <= q < Q)
 *               + beta * dx[n,c,h,w]
 *
 * on the handle's stream, asynchronously.  The cuDNN page ("Proposed
 * Method") names forward and backward routines and the maxDNN page
 * (Abstract, RQ4) the backward pass, without a formula; this is the plain
 * reading.
 *
 * The geometry is the forward problem's: dx_desc plays x (N, C, H, W),
 * w_desc the packed K,C,R,S filter, conv its padding and strides, and
 * dy_desc must have the forward output dims (N, K, P, Q).  Element types
 * (dy, w, dx): (F32, F32, F32), (F64, F64, F64), (BF16, BF16, F32).  dy and
 * dx are device memory with any element strides; alpha, beta, beta == 0,
 * ownership, overlap and size rules as for mic_conv_forward.  No workspace.
 *
 * Errors: MIC_STATUS_BAD_PARAM (null handle/descriptor/pointer, unset
 * descriptor, dy dims not the forward output dims), MIC_STATUS_NOT_SUPPORTED
 * (dtype combination, size limit), MIC_STATUS_LAUNCH_FAILED. */
mic_status mic_conv_backward_data(mic_handle handle, double alpha,
                                  mic_filter_desc w_desc, const void* w,
                                  mic_tensor_desc dy_desc, const void* dy,
                                  mic_conv_desc conv, double beta,
                                  mic_tensor_desc dx_desc, void* dx);

/* Name of the kernel variant mic_conv_backward_data would launch (host
 * only), as mic_conv_forward_kernel_name. */
mic_status mic_conv_backward_data_kernel_name(mic_handle handle, mic_filter_desc w_desc,
                                              mic_tensor_desc dy_desc, mic_conv_desc conv,
                                              mic_tensor_desc dx_desc, char* buf, size_t buflen);

/* ---------------------------------------------------------------- filter gradient */

/* dw <- alpha * wgrad(x, dy) + beta * dw: the backward pass with respect to
 * the filter, i.e. the adjoint of the forward sum in F,
 *
 *   dw[k,c,r,s] = alpha * sum_{n,p,q} dY(n, k, p, q) * X(n, c, p*u + r - pad_top, q*v + s - pad_left)
 *               + beta * dw[k,c,r,s]
 *
 * on the handle's stream, asynchronously (same reading of the pages as
 * mic_conv_backward_data).  The geometry is the forward problem's: x_desc
 * the input, dw_desc the packed K,C,R,S filter (its dtype is the output's),
 * conv the padding and strides; dy_desc must have the forward output dims
 * (N, K, P, Q).  Element types (x, dy, dw): (F32, F32, F32), (F64, F64,
 * F64), (BF16, BF16, F32).  x and dy with any element strides; dw packed.
 * alpha, beta, ownership and size rules as for mic_conv_forward.  No
 * workspace: the reduction over N*P*Q positions is split across at most two
 * workgroups.  With beta == 0 and dw tiles too few to fill the GPU, the call
 * first zeroes dw, then two workgroups per tile add alpha times their
 * partial sums into it with atomic adds; two terms added onto zero give the
 * same bits in either order, so the result is still deterministic (reruns
 * and any workgroup order bit-identical).  dw's prior contents are not read
 * when beta == 0.
 *
 * Errors: MIC_STATUS_BAD_PARAM (null handle/descriptor/pointer, unset
 * descriptor, dy dims not the forward output dims), MIC_STATUS_NOT_SUPPORTED
 * (dtype combination, size limit), MIC_STATUS_LAUNCH_FAILED. */
mic_status mic_conv_backward_filter(mic_handle handle, double alpha,
                                    mic_tensor_desc x_desc, const void* x,
                                    mic_tensor_desc dy_desc, const void* dy,
                                    mic_conv_desc conv, double beta,
                                    mic_filter_desc dw_desc, void* dw);

/* Name of the kernel variant mic_conv_backward_filter would launch (host
 * only), as mic_conv_forward_kernel_name. */
mic_status mic_conv_backward_filter_kernel_name(mic_handle handle, mic_tensor_desc x_desc,
                                                mic_tensor_desc dy_desc, mic_conv_desc conv,
                                                mic_filter_desc dw_desc, char* buf, size_t buflen);

/* ---------------------------------------------------------------- pooling */

/* Pooling forward pass (cuDNN page, "Proposed Method": pooling among the
 * library's routines; no formula printed, so the plain reading):
 *
 *   MIC_POOL_MAX:             max of X over the window positions inside the
 *                             H x W plane (padding never wins; 0 if none)
 *   MIC_POOL_AVG_INCLUDE_PAD: (sum of X over the positions inside) / (R*S)
 *   MIC_POOL_AVG_EXCLUDE_PAD: (sum over the positions inside) / (their
 *                             number; 0 if none)
 *   y[n,c,p,q] = alpha * that + beta * y[n,c,p,q]
 *
 * The window geometry is the convolution's: R x S window at (p*u - pad_top,
 * q*v - pad_left), output size by the same floor rule.  Channels are pooled
 * independently. */
typedef enum {
    MIC_POOL_MAX = 0,
    MIC_POOL_AVG_INCLUDE_PAD = 1,
    MIC_POOL_AVG_EXCLUDE_PAD = 2
} mic_pool_mode;

typedef struct mic_pool_desc_st* mic_pool_desc;

mic_status mic_pool_desc_create(mic_pool_desc* desc);
mic_status mic_pool_desc_destroy(mic_pool_desc desc);

/* Mode, window (>= 1), per-side padding (>= 0), strides (>= 1); else
 * MIC_STATUS_BAD_PARAM. */
mic_status mic_pool_desc_set(mic_pool_desc desc, mic_pool_mode mode, int window_h, int window_w,
                             int pad_top, int pad_bottom, int pad_left, int pad_right,
                             int stride_h, int stride_w);
mic_status mic_pool_desc_get(mic_pool_desc desc, mic_pool_mode* mode, int* window_h, int* window_w,
                             int* pad_top, int* pad_bottom, int* pad_left, int* pad_right,
                             int* stride_h, int* stride_w);

/* Output dims (N, C, P, Q), host only; MIC_STATUS_BAD_PARAM if a descriptor
 * is unset or the window exceeds the padded input. */
mic_status mic_pool_forward_output_dim(mic_pool_desc pool, mic_tensor_desc x_desc,
                                       int* n, int* c, int* p, int* q);

/* y <- alpha * pool(x) + beta * y on the handle's stream, asynchronously.
 * Element types (x, y): (F32, F32), (F64, F64), (BF16, F32).  x and y with
 * any element strides; y's dims must equal the output dims.  Ownership,
 * alpha/beta, beta == 0 and size rules as for mic_conv_forward.  No
 * workspace.  Errors: MIC_STATUS_BAD_PARAM (null handle/descriptor/pointer,
 * unset descriptor, shape mismatch), MIC_STATUS_NOT_SUPPORTED (dtype
 * combination, size limit), MIC_STATUS_LAUNCH_FAILED. */
mic_status mic_pool_forward(mic_handle handle, double alpha, mic_pool_desc pool,
                            mic_tensor_desc x_desc, const void* x, double beta,
                            mic_tensor_desc y_desc, void* y);

/* ------------------------------------------------------------------ batch-reduce GEMM
 *
 * Single-building-block page (Georganas et al.), "Proposed Method": the
 * batch-reduce GEMM multiplies a batch of A blocks by a batch of B blocks
 * and reduces all products into one C block:
 *
 *   C[i_m, i_n] <- alpha * sum_{i < batch} sum_{i_k < k} A_i[i_m, i_k] * B_i[i_k, i_n]
 *                  + beta * C[i_m, i_n]
 *
 * with A_i[i_m, i_k] = a[i*a_stride_batch + i_m*a_stride_m + i_k*a_stride_k],
 * B_i[i_k, i_n] = b[i*b_stride_batch + i_k*b_stride_k + i_n*b_stride_n] and
 * C[i_m, i_n] = c[i_m*c_stride_m + i_n*c_stride_n], strides in elements.
 * A fully-connected layer is one block product (batch 1, k = input
 * features) or its input features cut into batch blocks.
 *
 * Element types: dtype MIC_DTYPE_F32 (A, B, C fp32), MIC_DTYPE_F64 (all
 * fp64), MIC_DTYPE_BF16 (A, B bf16, C fp32, fp32 accumulation).  a, b, c are
 * device pointers owned by the caller, aligned to their element size; the
 * call is asynchronous on the handle's stream and keeps no reference.
 * beta == 0 writes C without reading it (NaN-safe).  m == 0 or n == 0 is a
 * no-op; k == 0 or batch == 0 gives C <- beta * C (a, b may then be null).
 * C must not overlap A or B; distinct (i_m, i_n) must have distinct C
 * offsets.  No workspace.  Errors: MIC_STATUS_BAD_PARAM (null handle or
 * needed pointer, negative size or stride, misaligned pointer, aliased C
 * elements), MIC_STATUS_NOT_SUPPORTED (unknown dtype, an operand's highest
 * element offset or batch*k reaching 2^30), MIC_STATUS_LAUNCH_FAILED. */
mic_status mic_brgemm(mic_handle handle, mic_dtype dtype, int m, int n, int k, int batch, double alpha,
                      const void* a, int64_t a_stride_batch, int64_t a_stride_m, int64_t a_stride_k,
                      const void* b, int64_t b_stride_batch, int64_t b_stride_k, int64_t b_stride_n,
                      double beta, void* c, int64_t c_stride_m, int64_t c_stride_n);

/* Name of the kernel variant mic_brgemm would launch for these sizes and
 * strides (pointers taken as 16-byte aligned), host only, NUL-terminated
 * into buf of buflen bytes; errors as mic_brgemm's size and stride checks,
 * MIC_STATUS_BAD_PARAM if the name does not fit. */
mic_status mic_brgemm_kernel_name(mic_handle handle, mic_dtype dtype, int m, int n, int k, int batch,
                                  int64_t a_stride_batch, int64_t a_stride_m, int64_t a_stride_k,
                                  int64_t b_stride_batch, int64_t b_stride_k, int64_t b_stride_n,
                                  int64_t c_stride_m, int64_t c_stride_n, char* buf, size_t buflen);

#ifdef __cplusplus
}
#endif

#endif /* MICONV_H */
