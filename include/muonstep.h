/*
 * muonstep.h -- C ABI of the MI355X (gfx950) Muon optimizer step and weight EMA.
 *
 * What is computed (pages cited by title and section):
 *   - "Record: L_ParallelResiduals_UNetSkips_DepthRecur_Muon_ 1.0901" (PR #1893),
 *     "Architecture and training stack": Muon on the matrix parameters with
 *     momentum 0.99 and matrix LR 0.022; weight EMA with decay 0.9965.
 *   - "Record: Combined 3-Layer Recurrence + Parallel Residuals + Polar Express +
 *     Brotli" (PR #1396), "Techniques Combined": MuonEq-R row normalisation before
 *     the Newton-Schulz iteration, a per-step NS coefficient schedule, WD 0.105.
 *   - "Record: Improved Parallel Residuals + Systems Optimization" (PR #1584),
 *     "Summary": one fused Muon step and one batched EMA over all parameters,
 *     with the optimizer's arithmetic unchanged.
 *
 * The pages do not print the equations; the library implements the plain
 * reading of Muon, per matrix W (rows x cols, row-major, PyTorch out x in):
 *   M' = mu*M + G;  U = G + mu*M' (nesterov) or U = M' (otherwise)
 *   U_i <- U_i / (||U_i||_2 + 1e-7) for every stored row i     (if row_norm)
 *   X0 = U / (||U||_F + 1e-7);  X0 <- X0^T if rows > cols
 *   for k < ns_steps, (a,b,c) = coeffs[k]:  A = X X^T;  X <- a X + (b A + c A A) X
 *   O = X (transposed back);  s = sqrt(max(1, rows/cols))
 *   W' = (1 - lr*wd) W - lr*s*O
 * and the EMA  E' = d*E + (1 - d)*P  over any list of fp32 tensors; AdamW for
 * the parameters that are not Muon matrices (adamw_step below).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to contiguous fp32 data on the
 *     current HIP device.  The library never allocates, frees or synchronises
 *     on these calls; all work is ordered on `stream` (a hipStream_t; NULL is
 *     the null stream) and runs asynchronously.  muon_step runs part of its
 *     work on an internal stream of default priority (one per device, created
 *     on first use), forked from `stream` with an event recorded there and
 *     joined back into it with a second event, so what it enqueues still runs
 *     after the caller's earlier work on `stream` and before the caller's later
 *     work.  Faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Host arrays (the tensor list, the coefficient table, the EMA lists) are
 *     read during the call only; the caller keeps ownership.
 *   - Every argument is validated on the host before anything is enqueued, so a
 *     call that returns an error has no side effect and needs no GPU.
 *   - Return value 0 on success, otherwise one of the MUON_ERR_* codes; the
 *     message of the last error on the calling thread is muon_last_error().
 *   - Results are deterministic: every sum is taken in a fixed order; the only
 *     atomics (the persistent chain's tile counters) order work, never values.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef MUONSTEP_H
#define MUONSTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_OK 0
#define MUON_ERR_INVALID_ARG (-1)   /* null pointer, bad size, non-finite scalar */
#define MUON_ERR_UNSUPPORTED (-2)   /* shape beyond the limits, aliasing buffers */
#define MUON_ERR_WORKSPACE (-3)     /* workspace missing or smaller than required */
#define MUON_ERR_HIP (-4)           /* a HIP runtime call or kernel launch failed */

#define MUON_MAX_NS_STEPS 16        /* rows of the coefficient table, at most */
#define MUON_MAX_SHORT_SIDE 8192    /* min(rows, cols) of a Muon matrix, at most */
#define MUON_MAX_LONG_SIDE 65536    /* max(rows, cols) of a Muon matrix, at most */
#define MUON_MAX_TENSORS 4096       /* tensors per call, at most */

#define MUON_NS_BF16 0              /* bf16 MFMA, fp32 accumulation; compensated below a short side of 192 */
#define MUON_NS_FP32 1              /* NS products on fp32 MFMA */
#define MUON_NS_BF16X3 2            /* bf16 MFMA with hi/lo compensation in every product */

/* One Muon matrix.  param and momentum are updated in place; grad is read only.
 * update_out is optional (NULL to skip): when set, the orthogonalised update O
 * (rows x cols, fp32, before the lr and shape scaling) is written there.
 * ema is optional (NULL to skip): when set, the weight EMA of this matrix is
 * advanced in the same pass that writes W':  ema = d*ema + (1-d)*W'  with
 * d = ema_decay of the call (the batched EMA of "Record: Improved Parallel
 * Residuals + Systems Optimization" (PR #1584), "Summary", folded into the
 * step; identical to ema_update on the post-step weights).  None of the
 * buffers of any tensor of a call may overlap. */
typedef struct muon_tensor_t {
    float* param;
    const float* grad;
    float* momentum;
    float* update_out;
    float* ema;
    int32_t rows;
    int32_t cols;
} muon_tensor_t;

/* Bytes of device workspace muon_step needs for this list of matrices and this
 * NS precision.  Depends only on the shapes.  Returns 0 if the arguments are
 * invalid (see muon_last_error()). */
size_t muon_workspace_size(const muon_tensor_t* tensors, int32_t n, int32_t ns_precision);

/* One Muon step on n matrices (the equations above).
 *   tensors       host array of n descriptors, 1 <= n <= MUON_MAX_TENSORS; the
 *                 library groups them by shape itself.
 *   lr, momentum, weight_decay   finite scalars (momentum is mu).
 *   nesterov, row_norm           0 or 1.
 *   ns_steps      0 <= ns_steps <= MUON_MAX_NS_STEPS; 0 gives O = X0.
 *   ns_coeffs     host array of ns_steps rows (a_k, b_k, c_k), row-major,
 *                 finite; may be NULL only when ns_steps == 0.
 *   ns_precision  MUON_NS_BF16, MUON_NS_FP32 or MUON_NS_BF16X3.  Every NS
 *                 product runs on MFMA with fp32 accumulation; X is carried to
 *                 ~16 significant bits (bf16 hi + lo) or in fp32.  MUON_NS_BF16
 *                 forms X X^T and B X from the bf16 hi parts only (and A A from
 *                 hi*hi in bf16 plus hi*lo + lo*hi on e4m3 operands) for
 *                 matrices whose short side is at least 192, and the
 *                 compensated products (hi*hi + hi*lo + lo*hi in bf16
 *                 everywhere) below that; MUON_NS_BF16X3 compensates every
 *                 matrix.
 *   ema_decay     EMA decay d for the tensors whose ema is set; finite, in [0, 1]
 *                 (checked on every call).
 *   workspace     device buffer of at least muon_workspace_size(...) bytes,
 *                 256-byte aligned; its contents on entry do not matter.
 *   stream        hipStream_t the step is ordered on (see the conventions
 *                 above for the internal stream it forks and joins).
 * NaN or Inf inside the tensors is not checked and propagates. */
int muon_step(const muon_tensor_t* tensors, int32_t n, float lr, float momentum,
              int32_t nesterov, float weight_decay, int32_t row_norm, int32_t ns_steps,
              const float* ns_coeffs, int32_t ns_precision, float ema_decay, void* workspace,
              size_t workspace_bytes, void* stream);

/* muon_step together with the weight EMA of n_extra more tensors -- the
 * parameters that are not Muon matrices (embeddings, gains) -- in one call:
 * "Record: Improved Parallel Residuals + Systems Optimization" (PR #1584),
 * "Summary": the fused Muon step and one batched EMA over all parameters;
 * "Record: L_ParallelResiduals_UNetSkips_DepthRecur_Muon_ 1.0901" (PR #1893),
 * "Architecture and training stack", EMA row.  The results are those of
 * muon_step(...) followed by ema_update(extra_ema, extra_params, extra_numel,
 * n_extra, ema_decay, stream): the extra tensors' EMA uses the call's
 * ema_decay and the extra parameters as they are (the Muon step does not touch
 * them).  Because the extra buffers are disjoint from the matrices', their EMA
 * is enqueued on the internal stream with the least Newton-Schulz work, where
 * it runs beside the last phases of the others instead of after them.
 *   extra_ema, extra_params, extra_numel  host arrays of n_extra entries, as
 *                 in ema_update; extra_ema[i] is updated in place.
 *   n_extra       0 <= n_extra <= MUON_MAX_TENSORS (0: exactly muon_step).
 * Every other argument as in muon_step.  No buffer of the extra list may
 * overlap another, any buffer of the matrices, or the workspace
 * (MUON_ERR_UNSUPPORTED); everything is validated before anything is
 * enqueued. */
int muon_step_ema(const muon_tensor_t* tensors, int32_t n, float lr, float momentum,
                  int32_t nesterov, float weight_decay, int32_t row_norm, int32_t ns_steps,
                  const float* ns_coeffs, int32_t ns_precision, float ema_decay,
                  float* const* extra_ema, const float* const* extra_params, const int64_t* extra_numel,
                  int32_t n_extra, void* workspace, size_t workspace_bytes, void* stream);

/* muon_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as muon_step, without the workspace: the
 * library's static device workspace of MUON_STATIC_WORKSPACE_BYTES (a
 * file-scope device array that each GPU the library runs on holds until the
 * process ends) takes its place.  Calls that need more workspace than that
 * (muon_workspace_size) fail with MUON_ERR_WORKSPACE before anything is
 * enqueued.  The call allocates nothing (no hipMalloc, no allocating library
 * routine).  Every call on one GPU shares that GPU's static workspace and it
 * keeps the last call's contents (which no call depends on): calls that
 * overlap in time on one GPU, on any streams, race and must be serialised by
 * the caller. */
#define MUON_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int muon_step_static(const muon_tensor_t* tensors, int32_t n, float lr, float momentum,
                     int32_t nesterov, float weight_decay, int32_t row_norm, int32_t ns_steps,
                     const float* ns_coeffs, int32_t ns_precision, float ema_decay, void* stream);

/* Weight EMA over n fp32 tensors: ema[i][j] = decay*ema[i][j] + (1-decay)*params[i][j]
 * for j < numel[i].  Defined by "Record: L_ParallelResiduals_UNetSkips_DepthRecur_
 * Muon_ 1.0901" (PR #1893), "Architecture and training stack", EMA row (an
 * exponential moving average of the weights with EMA_DECAY 0.9965, kept over
 * every parameter and applied before quantization), and batched over all
 * tensors in one pass as in "Record: Improved Parallel Residuals + Systems
 * Optimization" (PR #1584), "Summary" ("batched EMA").  The decay multiplies
 * the old average and (1 - decay) the current parameter; call it after the
 * optimizer step, on the post-step parameters.
 *   ema, params   host arrays of n device pointers; ema[i] is updated in place,
 *                 params[i] is read only and must not overlap any ema[j].
 *   numel         host array of n element counts, each >= 0 (0 is skipped).
 *   decay         finite, 0 <= decay <= 1.
 *   1 <= n <= MUON_MAX_TENSORS. */
int ema_update(float* const* ema, const float* const* params, const int64_t* numel, int32_t n,
               float decay, void* stream);

/* Exchange the contents of ema[i] and params[i] (numel[i] fp32 elements each),
 * bit for bit: the weight EMA becomes the live parameter set, as the step
 * before quantization and evaluation needs ("Record: L_ParallelResiduals_
 * UNetSkips_DepthRecur_Muon_ 1.0901" (PR #1893), "Architecture and training
 * stack", EMA row: the EMA is applied before quantization); a second call swaps
 * the training weights back.
 *   ema, params   host arrays of n device pointers (4-byte aligned), both
 *                 updated in place; no two buffers of the call may overlap.
 *   numel         host array of n element counts, each >= 0 (0 is skipped).
 *   1 <= n <= MUON_MAX_TENSORS.  Same conventions as ema_update. */
int ema_swap(float* const* ema, float* const* params, const int64_t* numel, int32_t n, void* stream);

/* One fp32 tensor of the AdamW update (any shape, numel elements, contiguous).
 * param, exp_avg and exp_avg_sq are updated in place; grad is read only.  ema is
 * optional (NULL to skip): when set, the tensor's weight EMA is advanced on the
 * updated parameter in the same pass (ema = d*ema + (1-d)*param').  None of the
 * buffers of any tensor of a call may overlap. */
typedef struct adamw_tensor_t {
    float* param;
    const float* grad;
    float* exp_avg;
    float* exp_avg_sq;
    float* ema;
    int64_t numel;
} adamw_tensor_t;

/* AdamW over n fp32 tensors: the optimizer of the embeddings and scalar
 * parameters ("Record: L_ParallelResiduals_UNetSkips_DepthRecur_Muon_ 1.0901"
 * (PR #1893), "Architecture and training stack", Optimizer row, which names
 * AdamW and gives no equations).  Per element, with t = step:
 *   p <- (1 - lr*wd) p
 *   m <- beta1 m + (1 - beta1) g;   v <- beta2 v + (1 - beta2) g^2
 *   p <- p - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * then, where ema is set, ema <- ema_decay*ema + (1 - ema_decay)*p.
 *   tensors     host array of n descriptors, 1 <= n <= MUON_MAX_TENSORS; tensors
 *               with numel == 0 are skipped (their pointers may be NULL).
 *   lr, weight_decay  finite.   beta1, beta2  in [0, 1).   eps  finite, >= 0
 *               (eps == 0 with a zero second moment gives NaN, as the formula does).
 *   step        >= 1, the count of AdamW steps including this one.
 *   ema_decay   finite, in [0, 1] (checked on every call).
 * Pointers are device pointers, 4-byte aligned (16-byte alignment takes the
 * vector path).  Validated on the host before anything is enqueued; enqueued
 * on stream, never synchronises, allocates nothing. */
int adamw_step(const adamw_tensor_t* tensors, int32_t n, float lr, float beta1, float beta2, float eps,
               float weight_decay, int32_t step, float ema_decay, void* stream);

/* How muon_step schedules the Newton-Schulz iterations of the matrices whose
 * products run in base-precision bf16 (MUON_NS_BF16, short side >= 192):
 *   MUON_NS_SCHEDULE_PHASES  one launch per phase (Gram, square, update) and
 *                            iteration, the shape groups spread over two
 *                            streams (the default);
 *   MUON_NS_SCHEDULE_CHAIN   one persistent launch for every iteration of
 *                            every such matrix, each matrix bound to one XCD,
 *                            tiles taken in dependency order per matrix.
 * Both compute the same products on the same operand types and store the
 * same planes; the chain's Gram and square tiles run 4 waves instead of two
 * K groups of 4 and its Frobenius sum uses 256 threads instead of 512, so the
 * fp32 sums are taken in another order: results agree within the same
 * tolerances of the float64 reference, not bit for bit.  The setting is library-wide
 * and part of the schedule signature below.  Returns the previous setting,
 * or MUON_ERR_INVALID_ARG for an unknown value.  The environment variable
 * MUON_CHAIN=1 selects the chain when the library loads.  Needs no GPU. */
#define MUON_NS_SCHEDULE_PHASES 0
#define MUON_NS_SCHEDULE_CHAIN 1
int muon_set_ns_schedule(int32_t schedule);

/* Introspection of muon_step's schedule cache.  muon_step derives every table
 * it needs from the tensor list (pointer validation, shape groups, workspace
 * layout, launch sets, the Newton-Schulz chain's binding of matrices to XCDs)
 * and caches the result under the call's signature: every descriptor field,
 * the precision, the workspace pointer and size.  A later call with the same
 * signature (and the same muon_set_ns_schedule setting) checks only its
 * scalars and enqueues.  Writes the number of
 * schedules built and of cache hits since the library was loaded (either
 * pointer may be NULL) and returns the number of schedules held (at most 8,
 * least recently used dropped first).  Needs no GPU. */
int muon_plan_cache_stats(int64_t* built, int64_t* hits);

/* Message of the last failed call on this thread ("" if none). */
const char* muon_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int muon_version(void);

/* Kernel timing hook for measurement tools.  When enabled (non-zero), every
 * kernel the library launches is bracketed by HIP events on its stream and its
 * duration is added to a per-kernel-name total once the caller calls
 * muon_profile_read (which synchronises on the recorded events).  Disabled by
 * default; enabling adds two event records per launch. */
int muon_profile_enable(int32_t enable);

/* Copy the per-kernel totals since the last reset into host arrays of length
 * cap: names (each at most 47 characters plus NUL, 48 bytes per entry),
 * launch counts and summed milliseconds.  Returns the number of kernels (which
 * may exceed cap), or a negative MUON_ERR_* code.  reset != 0 clears the totals. */
int muon_profile_read(char* names, int64_t* counts, double* total_ms, int32_t cap, int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* MUONSTEP_H */
