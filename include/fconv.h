/*
 * fconv.h -- fused forward 2-D convolution over NHWC tensors on AMD MI355X
 * (gfx950), with a vertical epilogue fused into the convolution kernel.
 *
 * What one run computes (all dtypes):
 *
 *   acc[n,ho,wo,k] = sum_{r<R, s<S, c<C} X(n, ho*sh - pt + r, wo*sw - pl + s, c)
 *                                       * w[r,s,c,k]
 *   X(n,i,j,c) = x[n,i,j,c] inside the image, 0 outside (zero padding)
 *
 * i.e. cross-correlation (no filter flip) of an NHWC input with an HWIO
 * filter, as TensorFlow conv_ops_fused_int8.cc (LaunchFusedConv2DOpCpuInt8Helper:
 * "input in NHWC and filter in HWIO") and MXNet cudnn_deconvolution-inl.h
 * (InitDescriptors: cross-correlation mode) define it.  The contraction is an
 * implicit GEMM: rows are output pixels, the reduction runs over (r, s, c) in
 * the column order of TensorFlow conv_grad_filter_ops.cc, Im2col, and the
 * patch matrix is never materialised.
 *
 * Epilogues (applied in registers; the accumulator never reaches memory):
 *
 *   int8 (TensorFlow conv_ops_fused_int8.cc, BiasActivationOutputKernel, the
 *   cuDNN 8 order), every step an fp32 operation:
 *       t = (float)acc                              (round to nearest even)
 *       t = t * conv_input_scale                    FCONV_OP_SCALE
 *       t = fmaf((float)side, side_input_scale, t)  FCONV_OP_SIDE (skipped if
 *                                                   side_input_scale == 0)
 *       t = t + bias[k]                             FCONV_OP_BIAS
 *       y = (int8)clamp(rint(t), RELU ? 0 : -128, 127)   FCONV_OP_RELU
 *   The int8 result is bit-exact with that definition.
 *
 *   bf16 / fp32 (MIOpen "Using the fusion API": operators apply in the order
 *   they are added; the CBNA row of its supported-fusion tables):
 *       t = acc (fp32 accumulation)
 *       t = t + bias[k]                                        FCONV_OP_BIAS
 *       t = gamma[k] * (t - mean[k]) / sqrt(var[k] + eps) + beta[k]
 *                                                              FCONV_OP_BN
 *       t = max(t, 0)                                          FCONV_OP_RELU
 *         or t > 0 ? t : alpha * t                             FCONV_OP_LEAKY_RELU
 *         or min(max(t, 0), alpha)                             FCONV_OP_CLIPPED_RELU
 *         or min(max(t, alpha), beta)                          FCONV_OP_CLAMP
 *       y = t (fp32) or bf16(t) rounded to nearest even
 *   (alpha, beta: fconv_args.activ_alpha / activ_beta.  The fusion tables
 *   list these activations without formulas; these are their plain
 *   readings.)
 *
 * Plan / args split (MIOpen "Using the fusion API": a plan holds the data
 * geometry and the ordered operators and is compiled once; the per-run
 * arguments -- weights, bias, scalars -- are kept apart so the plan can be
 * reused).  Kernels are compiled ahead of time for gfx950, so "compiling" is
 * the host-side resolution done by fconv_plan_create.
 *
 * Conventions for every call:
 *  - Status codes only; nothing aborts or throws across this interface.
 *  - Device pointers are HIP device addresses (e.g. a torch tensor's
 *    data_ptr() on the GPU).  `stream` is a hipStream_t passed as void*
 *    (NULL = the default stream).
 *  - The library never allocates device memory: the caller owns every buffer,
 *    including the workspace that holds the repacked filter.
 *  - A plan is a host object.  fconv_plan_run never modifies it, so
 *    concurrent runs of one plan on different streams are safe when each has
 *    its own workspace and output.  The one call that changes a plan is
 *    fconv_plan_autotune (it replaces the plan's kernel configuration and
 *    updates a process-wide cache); it must not overlap any other call on
 *    the same plan.
 */
#ifndef FCONV_H
#define FCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported entry points (the library is built with hidden visibility). */
#define FCONV_API __attribute__((visibility("default")))

typedef enum {
  FCONV_OK = 0,
  FCONV_ERR_INVALID_ARG = 1, /* NULL / non-positive / inconsistent argument  */
  FCONV_ERR_UNSUPPORTED = 2, /* valid request this library does not perform  */
  FCONV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required  */
  FCONV_ERR_MISALIGNED = 4,  /* a tensor pointer is not 16-byte aligned,    */
                             /* or a [K] vector not 4-byte aligned          */
  FCONV_ERR_DEVICE = 5       /* the HIP runtime reported an error           */
} fconv_status;

/* Element type of x, w and y.  The side input is always int8 and only exists
 * for FCONV_INT8; bias and batch-norm vectors are always fp32. */
typedef enum { FCONV_INT8 = 0, FCONV_BF16 = 1, FCONV_FP32 = 2 } fconv_dtype;

/* SAME: Ho = ceil(H / stride_h); total padding P = max(0, (Ho-1)*stride_h + R - H),
 * floor(P/2) on top and the rest at the bottom (likewise for columns), as in
 * TensorFlow conv_ops_fused_int8.cc, LaunchFusedConv2DOpGpuInt8Helper.
 * VALID: no padding, Ho = (H - R)/stride_h + 1; requires H >= R and W >= S. */
typedef enum { FCONV_PAD_SAME = 0, FCONV_PAD_VALID = 1 } fconv_padding;

/* Epilogue operators.  Accepted sequences (anything else is
 * FCONV_ERR_UNSUPPORTED at plan creation, as MIOpen reports unsupported
 * operator sequences when they are added):
 *   FCONV_INT8:       SCALE, [SIDE], BIAS, [RELU]
 *   FCONV_BF16/FP32:  [BIAS], [BN], [RELU | LEAKY_RELU | CLIPPED_RELU | CLAMP]
 *                     (each optional, this order) */
typedef enum {
  FCONV_OP_SCALE = 1,
  FCONV_OP_SIDE = 2,
  FCONV_OP_BIAS = 3,
  FCONV_OP_BN = 4,
  FCONV_OP_RELU = 5,
  FCONV_OP_LEAKY_RELU = 6,   /* bf16 / fp32 only */
  FCONV_OP_CLIPPED_RELU = 7, /* bf16 / fp32 only */
  FCONV_OP_CLAMP = 8         /* bf16 / fp32 only */
} fconv_op;

#define FCONV_MAX_OPS 8

/* Plan flag (int8 only): the cuDNN 7 order of the int8 epilogue that
 * TensorFlow conv_ops_fused_int8.cc names in BiasActivationOutputKernel:
 *     t = fmaf((float)acc, conv_input_scale, bias[k])   one rounding
 *     t = fmaf((float)side, side_input_scale, t)         (SIDE op)
 *     y = (int8)clamp(rint(t), RELU ? 0 : -128, 127)
 * instead of the cuDNN 8 order above. */
#define FCONV_DESC_CUDNN7_ORDER 1u

/* Geometry and operator sequence of a plan (all by value; copied at create).
 * N may be 0 (every run is then a no-op); H, W, C, K, R, S, strides >= 1.
 * Groups and dilation are always 1 (the fused op on the pages supports no
 * other value). `flags`: 0 or FCONV_DESC_CUDNN7_ORDER (int8 plans); any
 * other bit is FCONV_ERR_UNSUPPORTED. */
typedef struct {
  int32_t N, H, W, C, K, R, S;
  int32_t stride_h, stride_w;
  int32_t padding; /* fconv_padding */
  int32_t dtype;   /* fconv_dtype   */
  int32_t n_ops;
  int32_t ops[FCONV_MAX_OPS]; /* fconv_op values, in application order */
  uint32_t flags;
} fconv_desc;

typedef struct fconv_plan_s* fconv_plan;

/* Run flag: `w` is ignored and the workspace already holds the filter packed
 * by fconv_plan_pack_filter (or by an earlier run of the same plan). */
#define FCONV_RUN_FILTER_PREPACKED 1u

/* Per-run arguments.  All tensors dense and contiguous.
 *   x      device, NHWC [N][H][W][C] of the plan dtype (bf16 as raw 16-bit)
 *   w      device, HWIO [R][S][C][K] of the plan dtype
 *   bias   device, fp32 [K]                          (needed iff BIAS op)
 *   side   device, int8 NHWC [N][Ho][Wo][K]           (needed iff SIDE op)
 *   conv_input_scale, side_input_scale: fp32 scalars (SCALE / SIDE ops)
 *   conv_input_scales  NULL, or device fp32 [K]: one conv_input_scale per
 *          output channel, which replaces the scalar (TensorFlow
 *          conv_ops_fused_int8.cc slices a scale tensor of more than one
 *          element at the output channel); int8 plans only
 *   activ_alpha, activ_beta: arguments of the LEAKY_RELU / CLIPPED_RELU /
 *          CLAMP activation (finite; CLAMP needs alpha <= beta)
 *   bn_gamma, bn_beta, bn_mean, bn_var: device fp32 [K] (needed iff BN op)
 *   bn_eps: batch-norm epsilon
 *   y      device, NHWC [N][Ho][Wo][K] of the plan dtype; must not overlap
 *          x, w, side or the workspace (no in-place operation)
 *   workspace / workspace_bytes: device scratch of at least
 *          fconv_plan_workspace_size bytes; receives the repacked filter
 *   flags  0 or FCONV_RUN_FILTER_PREPACKED
 * Tensor pointers (x, w, side, y, workspace) must be 16-byte aligned; the
 * [K] vectors 4-byte aligned. */
typedef struct {
  const void* x;
  const void* w;
  const float* bias;
  const void* side;
  float conv_input_scale;
  float side_input_scale;
  const float* bn_gamma;
  const float* bn_beta;
  const float* bn_mean;
  const float* bn_var;
  float bn_eps;
  void* y;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;
  const float* conv_input_scales;
  float activ_alpha;
  float activ_beta;
} fconv_args;

/* Validates `desc`, resolves output size and padding, checks the operator
 * sequence, and picks the kernel variant and tiling for the shape.  On success
 * *out receives a new plan (release with fconv_plan_destroy).  Host only; no
 * device work.  Errors: FCONV_ERR_INVALID_ARG (NULL pointer, non-positive
 * size or stride, VALID with H < R or W < S), FCONV_ERR_UNSUPPORTED (unknown
 * dtype / padding, an operator sequence outside the accepted ones, non-zero
 * flags, or a tensor of 2^31 elements or more). */
FCONV_API fconv_status fconv_plan_create(const fconv_desc* desc, fconv_plan* out);

/* Output size and the resolved padding (top, bottom, left, right).  Any of
 * the output pointers may be NULL. */
FCONV_API fconv_status fconv_plan_output_dims(fconv_plan plan, int32_t* Ho, int32_t* Wo,
                                    int32_t pads_tblr[4]);

/* Bytes of workspace a run needs (the filter repacked K-major for the matrix
 * cores, zero-padded to whole tiles). */
FCONV_API fconv_status fconv_plan_workspace_size(fconv_plan plan, size_t* bytes);

/* Enqueues only the filter repack (HWIO -> the K-major tile layout the conv
 * kernel reads) into `workspace` on `stream`; a later run may then pass
 * FCONV_RUN_FILTER_PREPACKED, as inference with fixed weights does.  The
 * workspace contents are only meaningful to runs of plans with the same
 * C, K, R, S and dtype. */
FCONV_API fconv_status fconv_plan_pack_filter(fconv_plan plan, void* stream, const void* w,
                                    void* workspace, size_t workspace_bytes);

/* Enqueues the fused convolution on `stream` and returns; results are valid
 * once the stream has been synchronised.  Every argument check happens before
 * anything is enqueued, so an error return leaves the stream untouched.
 * Unless FCONV_RUN_FILTER_PREPACKED is set, the filter repack is enqueued
 * first.  A zero side_input_scale skips the side input (TensorFlow's output
 * kernel does the same), but `side` must still be given when the plan has a
 * SIDE op.  Errors: FCONV_ERR_INVALID_ARG (NULL plan/args, a needed pointer
 * NULL, y overlapping an input), FCONV_ERR_MISALIGNED, FCONV_ERR_WORKSPACE,
 * FCONV_ERR_DEVICE (launch failure). */
FCONV_API fconv_status fconv_plan_run(fconv_plan plan, void* stream, const fconv_args* args);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * run as fconv_plan_run, with args->workspace and args->workspace_bytes
 * ignored.  The run's scratch (the repacked filter, and for a full-size VALID
 * filter the reduction ranges' partial sums) lives in a device array
 * of FCONV_NO_ALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends; nothing is allocated or freed per call.  Every
 * call on one GPU shares that GPU's array and leaves the last call's contents
 * in it, so calls that overlap on one GPU (other streams, other threads)
 * race; FCONV_RUN_FILTER_PREPACKED reuses the filter the previous call on
 * that GPU packed, and is only meaningful when that call had a plan with the
 * same C, K, R, S and dtype and the same filter.  Errors: as fconv_plan_run;
 * FCONV_ERR_WORKSPACE when the plan's workspace size exceeds
 * FCONV_NO_ALLOC_SCRATCH_BYTES; FCONV_ERR_DEVICE when the array's device
 * address cannot be obtained. */
#define FCONV_NO_ALLOC_SCRATCH_BYTES (4u << 20)
FCONV_API fconv_status fconv_plan_run_no_alloc(fconv_plan plan, void* stream,
                                               const fconv_args* args);

/* Autotuning, as TensorFlow (conv_ops_fused_int8.cc, the autotune path of
 * LaunchFusedConv2DOpGpuInt8Helper) and MXNet (cudnn_deconvolution-inl.h,
 * SelectAlgo) pick among algorithms by timing them and caching the choice per
 * problem key.  Times every kernel configuration that can run the plan's
 * shape (family and tiling), `repeats` launches each, on the caller's
 * buffers `args` (checked as by fconv_plan_run; y is overwritten and holds
 * the chosen configuration's result on return).  A candidate whose output
 * differs from the plan's own configuration (int8: any bit; bf16: normwise
 * 8e-3, about two ulps of the rounded output; fp32: 1e-5) is not chosen.
 * The fastest becomes the plan's configuration (the plan is modified) and is
 * cached for the process: later fconv_plan_create calls
 * with the same descriptor start from it (unless FCONV_FORCE_VARIANT pins a
 * family).  Synchronous: returns after the stream has drained.  Must not
 * run concurrently with other calls on the same plan.  *best_us (may be
 * NULL) receives the chosen configuration's time per launch.  Errors: as
 * fconv_plan_run; FCONV_ERR_INVALID_ARG for repeats outside 1..100000. */
FCONV_API fconv_status fconv_plan_autotune(fconv_plan plan, void* stream, const fconv_args* args,
                                           int32_t repeats, float* best_us);

/* Forget every autotuned configuration of this process. */
FCONV_API void fconv_autotune_cache_clear(void);

/* Frees the plan (host memory only).  NULL is a no-op. */
FCONV_API fconv_status fconv_plan_destroy(fconv_plan plan);

/* Name of the conv kernel the plan launches (for logs and profiles).  Static
 * storage; NULL for a NULL plan. */
FCONV_API const char* fconv_plan_kernel_name(fconv_plan plan);

/* Static, human-readable text for a status code. */
FCONV_API const char* fconv_status_string(fconv_status status);

/* ------------------------------------------------------------------------
 * Weight gradient (filter gradient) of the same convolution.
 *
 *   dw[r,s,c,k] = sum_{n<N, ho<Ho, wo<Wo} X(n, ho*sh - pt + r, wo*sw - pl + s, c)
 *                                          * dy[n,ho,wo,k]
 *
 * with X, the strides and the SAME/VALID padding exactly as in the forward
 * convolution above.  TensorFlow conv_grad_filter_ops.cc
 * (Conv2DCustomBackpropFilterOp) computes it per image as the Im2col patch
 * matrix transposed times the output gradient, [R*S*C, Ho*Wo] x [Ho*Wo, K],
 * summed over the images; here it is one implicit GEMM whose reduction runs
 * over all N*Ho*Wo output pixels, the patch matrix never materialised.
 *
 * The plan is created from an fconv_desc that describes the forward
 * convolution (N, H, W, C, K, R, S, strides, padding, dtype); n_ops must be 0.
 * dtype FCONV_BF16 or FCONV_FP32 (FCONV_INT8 is FCONV_ERR_UNSUPPORTED: the
 * int8 op has no gradient on the pages).  Products are exact and sums are
 * fp32 (matrix-core accumulation, then a fixed-order sum over pixel ranges),
 * so the result is deterministic: the same inputs give the same bits on every
 * run.  dw is written in the plan dtype (bf16 rounded to nearest even), or in
 * fp32 for a bf16 plan created with FCONV_WGRAD_OUT_FP32.
 * ------------------------------------------------------------------------ */

typedef struct fconv_wgrad_plan_s* fconv_wgrad_plan;

/* Descriptor flag of fconv_wgrad_plan_create: a bf16 plan writes dw as fp32
 * (the fp32 sums, unrounded).  No effect on an fp32 plan. */
#define FCONV_WGRAD_OUT_FP32 1u

/* Validates the descriptor and resolves Ho, Wo and the padding as
 * fconv_plan_create does; picks the tiling and how many pixel ranges the
 * reduction is split into.  Host only.  Errors: FCONV_ERR_INVALID_ARG (NULL
 * pointer, non-positive size or stride, VALID with H < R or W < S),
 * FCONV_ERR_UNSUPPORTED (dtype not bf16/fp32, n_ops != 0, unknown flags, x or
 * dy of 2 GiB or more). */
FCONV_API fconv_status fconv_wgrad_plan_create(const fconv_desc* desc, fconv_wgrad_plan* out);

/* Shape of dy, [N][Ho][Wo][K], and the resolved padding (top, bottom, left,
 * right).  Any output pointer may be NULL. */
FCONV_API fconv_status fconv_wgrad_plan_output_dims(fconv_wgrad_plan plan, int32_t* Ho,
                                                    int32_t* Wo, int32_t pads_tblr[4]);

/* Bytes of workspace a run needs: the fp32 partial sums of the pixel ranges
 * (0 when the reduction is not split). */
FCONV_API fconv_status fconv_wgrad_plan_workspace_size(fconv_wgrad_plan plan, size_t* bytes);

/* Enqueues dw = the weight gradient on `stream` and returns.
 *   x   device, NHWC [N][H][W][C] of the plan dtype
 *   dy  device, NHWC [N][Ho][Wo][K] of the plan dtype
 *   dw  device, HWIO [R][S][C][K], plan dtype or fp32 (FCONV_WGRAD_OUT_FP32);
 *       overwritten (zeros when N == 0); must not overlap x, dy or the
 *       workspace
 *   workspace / workspace_bytes: device scratch of at least
 *       fconv_wgrad_plan_workspace_size bytes (may be NULL when that is 0)
 * Pointers 16-byte aligned.  All checks happen before anything is enqueued.
 * Errors: FCONV_ERR_INVALID_ARG (NULL plan or tensor, overlap),
 * FCONV_ERR_MISALIGNED, FCONV_ERR_WORKSPACE, FCONV_ERR_DEVICE. */
FCONV_API fconv_status fconv_wgrad_plan_run(fconv_wgrad_plan plan, void* stream, const void* x,
                                            const void* dy, void* dw, void* workspace,
                                            size_t workspace_bytes);

/* Name of the main kernel the plan launches; NULL for a NULL plan. */
FCONV_API const char* fconv_wgrad_plan_kernel_name(fconv_wgrad_plan plan);

/* Frees the plan (host memory only).  NULL is a no-op. */
FCONV_API fconv_status fconv_wgrad_plan_destroy(fconv_wgrad_plan plan);

#ifdef __cplusplus
}
#endif

#endif /* FCONV_H */
