/*
 * libaddrmsnorm_dq — fused (Add)RmsNorm + per-row symmetric dynamic
 * quantization for AMD Instinct MI355X (gfx950).
 *
 * Operators (Huawei Ascend CANN operator pages, read as specification):
 *
 *  AddRmsNormDynamicQuantV2 — "aclnnAddRmsNormDynamicQuantV2", Formula:
 *      x        = x1 + x2                                  (xOut)
 *      y        = x / Rms(x) * gamma + beta,  Rms(x) = sqrt(mean_j x_j^2 + epsilon)
 *      input_k  = y * smoothScale_k   (y when smoothScale_k is absent)
 *      scale_k  = row_max(|input_k|) / 127  (INT8 output)  or  / 7  (INT4 output)
 *      y_k      = round(input_k / scale_k)
 *    Mean and max run over the last dimension (length n) of each row.
 *
 *  RmsNormDynamicQuant — "aclnnRmsNormDynamicQuant", formula section: the
 *    same without the add and without xOut, one quantized output and an
 *    optional smoothScales vector.
 *
 * Readings where the pages leave the arithmetic open (fixed by this
 * library): the add and all later steps run in fp32 on the unrounded sum;
 * only stored values are rounded (xOut to the input type, round to nearest
 * even; scales to fp32); round() is round-half-to-even; codes lie in
 * [-127, 127] or [-7, 7]; a row whose maximum is 0 gets scale 0 and codes 0;
 * epsilon is applied as the nearest fp32 value; beta absent = 0.
 *
 * Calling convention (the pages' two-phase form, "aclnnXxxGetWorkspaceSize"
 * then "aclnnXxx"): phase 1 validates every argument synchronously on the
 * host, chooses the kernel, and returns the workspace size and an executor;
 * phase 2 enqueues the work on a HIP stream and returns without waiting.
 *
 * Tensors: `adq_tensor` describes caller-owned DEVICE memory, dense
 * row-major ("ND" in the pages' Constraints), up to 8 dimensions.  The
 * library keeps the pointers inside the executor: the caller must keep the
 * memory alive and unchanged in place until the phase-2 work has finished.
 * Leading dimensions are flattened to rows M; the last dimension is n.
 *
 * Dtypes: x1, x2, xOut, gamma, beta, smooth scales: one of ADQ_F16 or
 * ADQ_BF16 (all the same).  Scales: ADQ_F32.  Quantized outputs: ADQ_INT8
 * (shape [..., n]) or ADQ_INT4X2 (shape [..., n/2], n even; byte j of a row
 * holds column 2j in its low nibble and column 2j+1 in its high nibble, each
 * a 4-bit two's complement code).  Each output's dtype selects its Q.
 *
 * Errors: every call returns an adq_status; adq_last_error() returns a
 * thread-local message for the last non-OK status of the calling thread.
 * Phase 2 never allocates and never synchronizes.
 *
 * Threads: phase-1 calls and executors may be used from any threads at
 * once; an executor may be run any number of times, on any streams.
 * Phase-2 calls that share a workspace must be ordered by the caller.
 *
 * Graphs: every phase-2 call may be captured into a HIP graph and the graph
 * replayed; no call records a memset, and no kernel keeps state between
 * launches (a split-row call captured on a stream runs its plain-launch
 * form, whose results are the same bits as the one-launch form's).
 *
 * Determinism: results are bitwise reproducible run to run (fixed
 * reduction order, no floating-point atomics), as the pages' Constraints
 * sections require of both operators.
 */
#ifndef ADQ_H
#define ADQ_H

#include <stdbool.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum adq_dtype {
  ADQ_F16 = 1,
  ADQ_BF16 = 2,
  ADQ_F32 = 3,
  ADQ_INT8 = 4,
  ADQ_INT4X2 = 5, /* two INT4 codes per byte, even column in the low nibble */
  ADQ_INT32 = 6   /* adapter indices of AddLora */
} adq_dtype;

#define ADQ_MAX_DIMS 8

/* A caller-owned, contiguous, row-major device tensor. */
typedef struct adq_tensor {
  void* data;     /* device address; must not be NULL for a present tensor */
  int32_t dtype;  /* adq_dtype */
  int32_t ndim;   /* 1 .. ADQ_MAX_DIMS (0 allowed for a scale of one row) */
  int64_t shape[ADQ_MAX_DIMS];
} adq_tensor;

typedef enum adq_status {
  ADQ_OK = 0,
  ADQ_ERR_NULLPTR = 1,       /* a required tensor, its data, or an out-pointer is NULL */
  ADQ_ERR_PARAM_INVALID = 2, /* shape, dtype pairing, empty tensor, mask rule, ... */
  ADQ_ERR_UNSUPPORTED = 3,   /* a dtype outside the supported set */
  ADQ_ERR_WORKSPACE = 4,     /* phase 2: workspace missing or smaller than phase 1 said */
  ADQ_ERR_RUNTIME = 5        /* no usable HIP device, or a HIP launch error */
} adq_status;

/* Opaque, library-owned plan of one call; reusable for repeated launches
 * with the same tensors until adq_executor_destroy(). */
typedef struct adq_executor adq_executor;

/*
 * AddRmsNormDynamicQuantV2, phase 1.
 *
 * x1, x2        [..., n] F16 or BF16, same shape and dtype; required.
 * gamma         [n] same dtype; required.
 * beta          [n] same dtype, or NULL (beta = 0).
 * smooth_scale1 [n] same dtype, or NULL.  smooth_scale2 likewise.
 * epsilon       added to mean(x^2) inside the square root.
 * output_mask   NULL (outputMaskOptional absent) or bool[2].
 * y1_out, y2_out      [..., n] ADQ_INT8 or [..., n/2] ADQ_INT4X2.
 * scale1_out, scale2_out  F32 with M elements (shape [...] or [M]).
 * x_out         [..., n] same dtype as x1; required.
 * workspace_size, executor: out-pointers; *executor must later be passed to
 *               adq_executor_destroy().
 *
 * Which outputs are produced ("aclnnAddRmsNormDynamicQuantV2", Formula
 * cases and Constraints):
 *   output_mask given: y1/scale1 iff mask[0], y2/scale2 iff mask[1];
 *     rejected (ADQ_ERR_PARAM_INVALID) when smooth_scale1 is given and
 *     mask[0] is false, when smooth_scale2 is given and mask[1] is false,
 *     or when both flags are false.
 *   output_mask NULL: y1/scale1 always; y2/scale2 iff both smooth scales
 *     are given; rejected when smooth_scale2 is given without smooth_scale1.
 * An output that is produced needs its tensors (else ADQ_ERR_NULLPTR).  An
 * output that is not produced may be NULL; if given, it is never written.
 * Empty tensors (a zero dimension) are rejected ("aclnnRmsNormDynamicQuant",
 * Constraints: no empty input or output).  A produced output that shares
 * memory with an input or with another produced output is rejected
 * (ADQ_ERR_PARAM_INVALID): some paths read x1 and x2 again after writing
 * xOut and the codes.
 */
adq_status adq_add_rms_norm_dynamic_quant_v2_get_workspace_size(
    const adq_tensor* x1, const adq_tensor* x2, const adq_tensor* gamma,
    const adq_tensor* beta, const adq_tensor* smooth_scale1, const adq_tensor* smooth_scale2,
    double epsilon, const bool* output_mask, const adq_tensor* y1_out,
    const adq_tensor* y2_out, const adq_tensor* scale1_out, const adq_tensor* scale2_out,
    const adq_tensor* x_out, uint64_t* workspace_size, adq_executor** executor);

/*
 * AddRmsNormDynamicQuantV2, phase 2: enqueue the work on `hip_stream` (a
 * hipStream_t; NULL = the default stream of the executor's device).
 * `workspace` is caller-owned device memory of at least the phase-1 size
 * (may be NULL when that size is 0), 8-byte aligned, with any contents: the
 * split-row path (ADQ_PATH_SPLIT) keeps its per-chunk partial sums and
 * maxima there between its launches, and every value it reads was written
 * by an earlier launch of the same call.  Concurrent launches that share a
 * workspace must be ordered by the caller.  Returns without waiting.
 */
adq_status adq_add_rms_norm_dynamic_quant_v2(void* workspace, uint64_t workspace_size,
                                             adq_executor* executor, void* hip_stream);

/*
 * AddRmsNormDynamicQuantV2, phase 2 without a workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving
 * loops that may not allocate, harnesses that forbid allocation.  Runs
 * `executor` exactly as adq_add_rms_norm_dynamic_quant_v2 does (same
 * kernels, same results bit for bit), but the split-row path's partial
 * results go to a buffer of ADQ_STATIC_SCRATCH_BYTES that the library keeps
 * in each device's memory (a static device array, held until the process
 * ends) instead of a caller's workspace.  Allocates nothing.  Returns
 * ADQ_ERR_WORKSPACE when the executor needs a larger workspace than that
 * buffer (the plan's workspace size, as phase 1 reported it),
 * ADQ_ERR_PARAM_INVALID for an executor of another operator, and
 * ADQ_ERR_RUNTIME when the buffer's address cannot be found (it is looked up
 * once per device, on the first call there that needs it).  All calls on one
 * device share the one buffer, which keeps the last call's contents (nothing
 * in it needs clearing): calls that may run at the same time on one device
 * (on different streams, or graphs replayed concurrently) race, and the
 * caller must order them.
 */
#define ADQ_STATIC_SCRATCH_BYTES (1u << 20)
adq_status adq_add_rms_norm_dynamic_quant_v2_no_alloc(adq_executor* executor, void* hip_stream);

/*
 * RmsNormDynamicQuant, phase 1.
 * x [..., n] F16/BF16; gamma [n]; beta [n] or NULL; smooth_scales [n] or
 * NULL; y_out [..., n] ADQ_INT8 or [..., n/2] ADQ_INT4X2; scale_out F32
 * with M elements.  Same validation and errors as the V2 call.
 */
adq_status adq_rms_norm_dynamic_quant_get_workspace_size(
    const adq_tensor* x, const adq_tensor* gamma, const adq_tensor* beta,
    const adq_tensor* smooth_scales, double epsilon, const adq_tensor* y_out,
    const adq_tensor* scale_out, uint64_t* workspace_size, adq_executor** executor);

/* RmsNormDynamicQuant, phase 2; as adq_add_rms_norm_dynamic_quant_v2. */
adq_status adq_rms_norm_dynamic_quant(void* workspace, uint64_t workspace_size,
                                      adq_executor* executor, void* hip_stream);

/*
 * INT8 x INT8 GEMM with per-row and per-column scales: the consumer of the
 * quantized activations.  With y1Out = round(input1 / scale1Out) (the V2
 * Formula), input1 ~ y1Out * scale1Out row by row, and a linear layer whose
 * weights are quantized per output column (w ~ w_q * w_scale) computes
 *
 *   out[..., j] = (sum_k a[..., k] * w[j, k]) * a_scale[...] * w_scale[j] + bias[j]
 *
 * a        [..., k] ADQ_INT8, row-major, 16-byte aligned (e.g. y1_out)
 * a_scale  F32 with one value per row of a (e.g. scale1_out), 4-byte aligned
 * w        [n, k] ADQ_INT8, row-major (each output's weights contiguous), 16-byte aligned
 * w_scale  [n] F32, 4-byte aligned
 * bias     [n] F32 (4-byte aligned), or NULL
 * out      [..., n] F32, BF16 or F16 (rounded to nearest even from fp32)
 * k must be a multiple of 16 and at most 131072 (the integer sum stays in
 * int32); n at most 1048576.  The integer sum is exact; the epilogue is
 * ((float)sum * a_scale) * w_scale + bias in fp32.  Workspace size is 0.
 * Errors as for the other phase-1 calls.
 */
adq_status adq_w8a8_gemm_get_workspace_size(const adq_tensor* a, const adq_tensor* a_scale,
                                            const adq_tensor* w, const adq_tensor* w_scale,
                                            const adq_tensor* bias, const adq_tensor* out,
                                            uint64_t* workspace_size, adq_executor** executor);

/* GEMM phase 2; as adq_add_rms_norm_dynamic_quant_v2. */
adq_status adq_w8a8_gemm(void* workspace, uint64_t workspace_size, adq_executor* executor,
                         void* hip_stream);

/*
 * AddLora ("aclnnAddLora", Formulas): rows of x are grouped by their adapter
 * index; for each row b with g = indices[b] in [0, W)
 *
 *   Z1 = x[b, :] . weight_a[g, layer_idx]          (shrink, h1 -> rank)
 *   Z2 = Z1 . weight_b[g, layer_idx] * scale       (expand, rank -> h2)
 *   out[b, y_offset + j] = y[b, y_offset + j] + Z2[j],  j < y_slice_size
 *
 * and every other element of out equals y (rows with an index outside
 * [0, W) get no contribution).
 *
 * y          [..., h3] F16 or BF16
 * x          [..., h1] same dtype, same leading dimensions (rows) as y
 * weight_b   [W, L, rank, h2] same dtype, h2 == y_slice_size
 * indices    ADQ_INT32 with one value per row (any shape)
 * weight_a   [W, L, h1, rank] same dtype, or NULL: the shrink is skipped and
 *            Z1 = x[b, :] (then h1 must equal rank)
 * layer_idx  in [0, L); scale finite (applied as the nearest float);
 *            0 <= y_offset and y_offset + y_slice_size <= h3
 * out        same shape and dtype as y; either y itself (in place: only the
 *            slice of rows with an adapter is written) or memory that does
 *            not overlap y.
 * Arithmetic in fp32 (Z1 is not rounded between the two products; for BF16
 * at ranks 32, 64 and 128 the expand's sums run in the matrix unit, with Z1
 * entering as three bf16 pieces whose sum is exactly Z1); each slice value is
 * rounded once to the storage type.  W <= 2048, rank <= 1024.
 * Workspace: the tiled path (see adq_path) needs one, 8-byte aligned, whose
 * contents need not be initialised (tile table, grouped row order, partial
 * sums and, above 8192 rows, class counts per 8192 rows, all rewritten by
 * every launch before they are read; calls that share a workspace
 * must not overlap); the generic path needs none.  Errors as for the other
 * phase-1 calls.
 */
adq_status adq_add_lora_get_workspace_size(const adq_tensor* y, const adq_tensor* x,
                                           const adq_tensor* weight_b,
                                           const adq_tensor* indices,
                                           const adq_tensor* weight_a, int64_t layer_idx,
                                           double scale, int64_t y_offset,
                                           int64_t y_slice_size, const adq_tensor* out,
                                           uint64_t* workspace_size, adq_executor** executor);

/* AddLora phase 2; as adq_add_rms_norm_dynamic_quant_v2. */
adq_status adq_add_lora(void* workspace, uint64_t workspace_size, adq_executor* executor,
                        void* hip_stream);

/* Free an executor (NULL is a no-op).  Launched work is not affected. */
void adq_executor_destroy(adq_executor* executor);

/*
 * Kernel path of an executor.  ADQ_PATH_AUTO is chosen by phase 1 from the
 * shape; the others force a path (for tests and tuning).  ADQ_PATH_ROW:
 * one workgroup per row, 128-bit accesses (n % 8 == 0, 16-byte aligned
 * tensors, n <= 65536).  ADQ_PATH_SPLIT: S workgroups per row, each on a
 * chunk of the row, handing the per-chunk partial sums of squares and
 * maxima over through the workspace, in one launch or in two or three per
 * batch of rows (see adq_executor_set_split; n % 8 == 0, 16-byte aligned
 * tensors; AUTO takes it for rows longer than 65536 columns, and for rows
 * of at least 4096 columns when there are at most a quarter as many rows
 * as compute units).
 * ADQ_PATH_GENERIC: any n and alignment.
 * GEMM executors: ADQ_PATH_GEMM_TILE128 (128 x 128 output tiles),
 * ADQ_PATH_GEMM_TILE256 (256 x 256 tiles) and ADQ_PATH_GEMM_TILE32 (32
 * columns and up to 128 rows per tile, K split over the wavefronts of the
 * workgroup, for few rows); AUTO takes the 32-column tiles for few rows,
 * else 256 once the 256-tiles cover the compute units, else 128.  Each
 * accepts any valid GEMM shape; the operator paths are rejected for a GEMM
 * executor and vice versa.
 * AddLora executors: AUTO (the tiled kernel when the shapes and alignments
 * allow it: h1 % 8 == 0, rank 8, 16, 32, 64 or 128, h2 a multiple of 4, h3 and
 * y_offset multiples of 8, aligned tensors, one weight_b[g, layer] under
 * 4 GiB and one weight_a[g, layer] under 2 GiB; a batch whose y or x reaches 4 GiB runs as consecutive launch
 * sequences over row ranges below it, on the same stream and workspace) or
 * ADQ_PATH_GENERIC (one workgroup per row, any shape).
 */
typedef enum adq_path {
  ADQ_PATH_AUTO = 0,
  ADQ_PATH_ROW = 1,
  ADQ_PATH_SPLIT = 2,
  ADQ_PATH_GENERIC = 3,
  ADQ_PATH_GEMM_TILE128 = 4,
  ADQ_PATH_GEMM_TILE256 = 5,
  ADQ_PATH_GEMM_TILE32 = 6
} adq_path;

/*
 * Re-plan `executor` for `path` and return its workspace size.  Returns
 * ADQ_ERR_PARAM_INVALID when the shape does not meet that path's
 * conditions (the executor is then unchanged).
 */
adq_status adq_executor_set_path(adq_executor* executor, int32_t path,
                                 uint64_t* workspace_size);

/*
 * Split-row geometry of an operator executor (AddRmsNormDynamicQuantV2 or
 * RmsNormDynamicQuant), for tests and tuning: moves it to ADQ_PATH_SPLIT
 * and returns the new workspace size.  ADQ_ERR_PARAM_INVALID leaves the
 * executor unchanged.
 *
 * splits    chunks per row, 0 = the planner's choice; otherwise a count that
 *           cuts n into whole chunks of at most 2048 8-column vectors, all
 *           but the last of one size (at most 64 for the one-launch form).
 * launches  0 = the planner's choice (one launch when all workgroups of the
 *           call fit on the chip at once, else two or three);
 *           1 = one kernel whose workgroups exchange their chunks' partial
 *           sums of squares and maxima through the workspace, each slot
 *           tagged with a value the host makes for the call; a wait for a
 *           slot ends after `wait_us` and the waiting workgroup then
 *           computes the missing partial result itself (same code, same
 *           bits), so results never depend on timing.  A call on a stream
 *           that is being captured into a graph runs the plain two- or
 *           three-launch form instead (a replay would repeat the tag);
 *           2 = plain kernels; the last takes each row's maxima over the
 *           whole row;  3 = plain kernels, one of them for the maxima.
 * wait_us   one-launch form: longest wait per exchange in microseconds
 *           (< 0: the default, 20; 0: one look, then compute what is missing).
 * spread    nonzero: a row's chunks go to workgroups on different XCDs.
 *
 * For one chunk count every form, wait and placement gives the same bits
 * (the row's sum of squares is added up chunk by chunk in the same order);
 * another chunk count adds it up in another order.
 */
typedef struct adq_split_config {
  int32_t splits;
  int32_t launches;
  int32_t wait_us;
  int32_t spread;
} adq_split_config;

adq_status adq_executor_set_split(adq_executor* executor, const adq_split_config* config,
                                  uint64_t* workspace_size);

/*
 * Write a one-line description of the plan (path, kernel variant, block,
 * grid) into buf (NUL-terminated, truncated to len).  Returns the chosen
 * path (adq_path), or -1 for a NULL executor.
 */
int32_t adq_executor_describe(const adq_executor* executor, char* buf, uint64_t len);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* adq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ADQ_H */
