/*
 * muon.h — C ABI of the MI355X (gfx950) Muon optimizer step.
 *
 * One Muon step updates every 2-D weight W (rows x cols = fan_out x fan_in,
 * row-major, fp32) from its gradient G and its momentum M:
 *
 *   M <- mu*M + G                          classic SGD momentum
 *   N  = mu*M + G                          Nesterov look-ahead on the new M
 *                                          (or the EMA style, see below)
 *   O' = HybridNewtonSchulz(N)             per NS unit (see below)
 *   W <- W*(1 - lr*wd) - lr*scale*O'       decoupled weight decay
 *
 * Sources (web pages, cited by title and section):
 *  - DeepSeek tech notes "Muon 优化器": section 1 Algorithm 1 (the step and
 *    the spectral scale sqrt(max(n, m))*gamma), section 2 (Frobenius
 *    normalisation; quintic step a*X + b*(X X^T) X + c*(X X^T)^2 X; hybrid
 *    schedule 8 x (3.4445, -4.7750, 2.0315) then 2 x (2, -1.5, 0.5); a zero
 *    matrix is left as zero), section 3 (momentum 0.95, weight decay 0.1,
 *    gamma 0.18) and the learning rate 2.7e-4 of the section-2 sketch.
 *  - RFC-0023 "对齐 MaxText Muon 优化器实现与 Megatron-LM 完整行为":
 *    方案 1 (SGD momentum with Nesterov on the updated buffer, no bias
 *    correction), background / 方案 3 (split_head: per-head units with
 *    fan_out = head_dim), 方案 4 (muon_batch_update: same-shape matrices are
 *    stacked and orthogonalised in one batched pass; muon_batch_update_size
 *    chunks each shape group).
 *  - Megatron-LM PR "Scaling for MuP over Muon optimizer": spectral scale
 *    sqrt(max(fan_in, fan_out)) and unit_rms_norm scale sqrt(fan_out/fan_in).
 *
 * An NS unit is a whole matrix, or one block of `split_rows` consecutive rows
 * of it (split_head).  Units are independent; their results do not depend on
 * how they are grouped, batched or chunked.
 *
 * Conventions for every entry point:
 *  - All data pointers are device pointers on the current HIP device and must
 *    be 16-byte aligned.  Hyper-parameter and descriptor structs are host
 *    pointers.
 *  - Work is enqueued on `stream` (0 = the null stream) and is asynchronous;
 *    the caller keeps every buffer alive until the stream has passed it.  No
 *    entry point synchronises the device or allocates device memory.
 *  - Every argument is validated before anything is launched; on any error
 *    other than MUON_ERR_HIP nothing has been written.
 *  - No C++ exception crosses this interface.
 */
#ifndef MUON_H_
#define MUON_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUON_OK = 0,
  MUON_ERR_NULL = -1,      /* a required pointer is NULL */
  MUON_ERR_SHAPE = -2,     /* rows/cols/batch < 1, split_rows not dividing rows, sizes too
                              large: one NS unit padded to the tile (256, or 128 when
                              min(rows, cols) < 256) must hold under 2^30 elements, the
                              launch grids stay under 2^30 workgroups, and one call makes
                              at most 2^20 stacked passes */
  MUON_ERR_DTYPE = -3,     /* unknown dtype / precision / scale enum */
  MUON_ERR_ALIGN = -4,     /* a data pointer is not 16-byte aligned */
  MUON_ERR_WORKSPACE = -5, /* workspace NULL or smaller than muon_workspace_size() */
  MUON_ERR_HYPER = -6,     /* invalid hyper-parameters (non-finite, bad stage table) */
  MUON_ERR_HIP = -7,       /* a HIP call failed; outputs are undefined */
  MUON_ERR_ALIAS = -8,     /* overlapping input/output buffers where not allowed */
  MUON_ERR_SCHEDULE = -9   /* an NS launch whose workgroups wait on each other
                              (persistent, or small units split on chip) stopped:
                              a wait ran out of time (reported only by
                              muon_workspace_status, never by the step calls);
                              outputs are undefined */
} muon_status;

typedef enum { MUON_DTYPE_F32 = 0, MUON_DTYPE_BF16 = 1 } muon_dtype;

typedef enum { MUON_SCALE_SPECTRAL = 0, MUON_SCALE_UNIT_RMS_NORM = 1 } muon_scale_mode;

/* Precision of the Newton-Schulz matrix products.  FP32: fp32 operands on
 * the fp32 matrix cores.  BF16: bf16 operands with fp32 accumulation.  What
 * is rounded (nearest-even) to bf16 is what the products read: the iterate
 * X (kept only in bf16), the Gram A (whose bf16 copy also feeds the b*A
 * term) and B' = a*I + b*A + c*A^2 (the quintic step regrouped as B'*X, so
 * a*X rides on B's diagonal).  The epilogues form their results in fp32
 * before rounding; the last iteration's output and the weight update stay
 * fp32. */
typedef enum { MUON_NS_FP32 = 0, MUON_NS_BF16 = 1 } muon_ns_precision;

/* How the Newton-Schulz of a stacked pass is run.  PERSISTENT and LAUNCHES
 * run the same tiled products and give bit-identical results.
 * PERSISTENT: one launch runs every iteration of the pass.  Workgroups claim
 *   output tiles in order (for each iteration: the Gram tiles of every
 *   unit, then the polynomial tiles, then the apply tiles) and each tile
 *   waits until its unit has finished the products before it, so tiles of
 *   different units and products overlap.  A wait is bounded (a few seconds
 *   of wall clock); if one ever runs out the launch stops and
 *   muon_workspace_status reports MUON_ERR_SCHEDULE.
 * LAUNCHES: one launch per product and iteration, in stream order.
 * AUTO (default): per pass, whichever is faster on the MI355X.
 *   - Wide units (rows < cols) of at most 128 x 128 (fp32 products: at most
 *     64 rows) take the whole step, momentum to update, in one launch of
 *     one workgroup per unit.
 *   - Other wide units of at most 128 rows with bf16 products run their NS
 *     on chip (A and B' in the workgroup, one pass over X per iteration):
 *     one workgroup per unit when the units span at most eight 128-column
 *     blocks or number at least half the CUs, else each unit split over
 *     several workgroups that sum their partial Grams through memory
 *     (those waits are bounded like PERSISTENT's).
 *   - Other passes of units with min(rows, cols) < 256, and passes of a
 *     single unit, use LAUNCHES; the rest PERSISTENT.  A single-unit pass
 *     with min(rows, cols) >= 256 instead runs inside the PERSISTENT
 *     launch of another pass of the call whose units have the same
 *     orientation (with bf16 products; any with fp32 ones), when that pass
 *     takes one claim queue on the device (fewer units than XCCs, or
 *     units that do not spread evenly over them); its tiles then fill the
 *     CUs that the other pass leaves idle.  The workspace holds both
 *     passes' buffers for such a pair.
 *   The on-chip kernels round like the tiled products (bf16 operands, fp32
 *   accumulation) but in another order (b*A from A's fp32 accumulator; the
 *   one-launch step also adds a*X from the fp32 iterate), so results agree
 *   with a forced schedule to rounding. */
typedef enum {
  MUON_SCHEDULE_AUTO = 0,
  MUON_SCHEDULE_PERSISTENT = 1,
  MUON_SCHEDULE_LAUNCHES = 2
} muon_schedule;

/* Momentum and look-ahead rule (RFC-0023 方案 1, both styles):
 * SGD: M <- mu*M + G;            N = mu*M + G (on the updated M)
 * EMA: M <- mu*M + (1 - mu)*G;   N = mu*bc(M, t+1) + (1 - mu)*bc(G, t),
 *      bc(x, k) = x / (1 - mu^k), t = muon_hyper.step (1-based), 0 <= mu < 1.
 * NS is invariant to the scale of its input, so the EMA style differs from
 * the SGD style only through the bias corrections. */
typedef enum { MUON_NESTEROV_SGD = 0, MUON_NESTEROV_EMA = 1 } muon_nesterov_style;

/* A bank of `batch` equal-shape matrices stored back to back (stride
 * rows*cols elements).  rows = fan_out, cols = fan_in.  split_rows = 0: each
 * matrix is one NS unit; otherwise rows % split_rows == 0 and every block of
 * split_rows rows is a unit with fan_out = split_rows (split_head). */
typedef struct {
  int64_t batch;
  int64_t rows;
  int64_t cols;
  int64_t split_rows;
  int32_t grad_dtype; /* muon_dtype of the gradient (muon_step_batched only) */
  int32_t reserved;   /* must be 0 */
} muon_matrix_desc;

/* `steps` quintic steps with coefficients (a, b, c). */
typedef struct {
  int32_t steps;
  float a, b, c;
} muon_ns_stage;

#define MUON_MAX_STAGES 4

typedef struct {
  float lr;                  /* eta */
  float mu;                  /* momentum */
  float weight_decay;        /* lambda (decoupled) */
  float gamma;               /* spectral-scale multiplier */
  int32_t scale_mode;        /* muon_scale_mode */
  int32_t ns_precision;      /* muon_ns_precision */
  int32_t batch_update_size; /* max NS units per stacked pass; 0 = whole shape group */
  int32_t n_stages;          /* 1..MUON_MAX_STAGES */
  muon_ns_stage stages[MUON_MAX_STAGES];
  int32_t schedule;          /* muon_schedule */
  int32_t nesterov_style;    /* muon_nesterov_style */
  int32_t step;              /* 1-based index of this step (EMA style only) */
  int32_t reserved;          /* must be 0 */
} muon_hyper;

/* Fill `h` with the pages' values: lr 2.7e-4, mu 0.95, weight_decay 0.1,
 * gamma 0.18, spectral scale, bf16 NS products, whole-group batches, and the
 * hybrid schedule 8 x (3.4445, -4.7750, 2.0315) + 2 x (2, -1.5, 0.5)
 * (DeepSeek tech notes "Muon 优化器" sections 1-3); SGD-style momentum,
 * step 1, AUTO schedule.  NULL is ignored. */
void muon_hyper_default(muon_hyper* h);

/* Bytes of device workspace that muon_step_batched / muon_newton_schulz_batched
 * need for these matrices and hyper-parameters (the same value for both).
 * The workspace holds a status word, the NS iterates, Gram and polynomial
 * matrices of the largest stacked pass, the per-unit norms and the schedule
 * counters; it is scratch, owned by the caller, and may be reused freely
 * between calls on the same stream (calls that share a workspace must not
 * run concurrently).
 * Errors: MUON_ERR_NULL, MUON_ERR_SHAPE, MUON_ERR_DTYPE, MUON_ERR_HYPER. */
int muon_workspace_size(const muon_matrix_desc* mats, int64_t n_mats, const muon_hyper* h,
                        size_t* bytes);

/* One Muon step over `n_mats` banks (DeepSeek tech notes "Muon 优化器"
 * section 1 Algorithm 1 with the section-2 hybrid Newton-Schulz; RFC-0023
 * 方案 1 momentum (either style), split_head and 方案 4 batching; Megatron-LM PR "Scaling
 * for MuP over Muon optimizer" scale modes).
 *   params[i]  : float*  (batch, rows, cols)   W, updated in place
 *   grads[i]   : bf16 or fp32 (batch, rows, cols), read only
 *   momenta[i] : float*  (batch, rows, cols)   M, updated in place
 * A unit whose Nesterov look-ahead is exactly zero gets O' = 0, i.e. only
 * the weight decay.  Buffers of different banks must not overlap, and a
 * bank's params, grads and momenta must be distinct.  n_mats = 0 is a no-op.
 * The call only enqueues kernels on `stream` (the first call on a device
 * also queries the device), and every kernel resets the counters it uses by
 * its own writes, so a call made while `stream` is being captured into a HIP
 * graph replays like a fresh call on the same buffers.
 * Errors: every code above. */
int muon_step_batched(float* const* params, const void* const* grads, float* const* momenta,
                      const muon_matrix_desc* mats, int64_t n_mats, const muon_hyper* h,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Hybrid Newton-Schulz only (DeepSeek tech notes "Muon 优化器" section 2):
 * for every unit of x_in[i] (fp32, (batch, rows, cols)) writes the
 * unscaled NS output O' to o_out[i] (fp32, same shape); a zero unit gives
 * zeros.  x_in[i] and o_out[i] may be the same buffer.  grad_dtype of the
 * descriptors is ignored; h->ns_precision, stages and batch_update_size
 * apply.  Errors: every code above. */
int muon_newton_schulz_batched(const float* const* x_in, float* const* o_out,
                               const muon_matrix_desc* mats, int64_t n_mats, const muon_hyper* h,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* muon_step_batched without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc).  The library's own fixed device scratch
 * of 128 MiB per GPU (held until the process ends) takes the workspace's
 * place; nothing is allocated on any call.  Arguments, results and the
 * other errors are those of muon_step_batched.  Differences:
 *  - MUON_ERR_WORKSPACE when the step needs more scratch than 128 MiB (the
 *    size muon_workspace_size reports), before anything runs;
 *  - every tiled pass runs as one launch per product (the schedule's
 *    PERSISTENT and AUTO choice of it do not apply), whose kernels never
 *    wait, so there is no stopped launch to report; results are bit-identical
 *    to muon_step_batched's;
 *  - all calls on one GPU share its scratch: calls that overlap on one GPU
 *    (on different streams, or from several threads) race and give
 *    undefined results; the caller orders them. */
int muon_step_batched_noalloc(float* const* params, const void* const* grads,
                              float* const* momenta, const muon_matrix_desc* mats, int64_t n_mats,
                              const muon_hyper* h, hipStream_t stream);

/* Kernel classes that a trace can bracket. */
typedef enum {
  MUON_KERNEL_MOMENTUM = 1, /* momentum + Nesterov + Frobenius partial sums */
  MUON_KERNEL_NORMALIZE = 2,/* norm finish (+ X0 = N/||N|| on the fp32 path;
                               the tiled bf16 path folds 1/||N|| into its
                               first iteration) */
  MUON_KERNEL_GRAM = 3,     /* A = X X^T on the smaller side */
  MUON_KERNEL_POLY = 4,     /* B' = a*I + b*A + c*A*A */
  MUON_KERNEL_APPLY = 5,    /* X <- B'*X (last one: the weight update) */
  MUON_KERNEL_NS = 6,       /* every NS product of a pass in one launch
                               (the persistent kernel) */
  MUON_KERNEL_NS_SMALL = 7  /* the whole NS of a pass of small units in one
                               launch (the on-chip kernel) */
} muon_kernel_kind;

/* Timing hook: when passed to the *_traced entry points, every launch of
 * kernel class `kind` is bracketed by hipEventRecord(events[2k]) and
 * hipEventRecord(events[2k+1]) on the step's stream, for k = 0 .. capacity-1;
 * `count` returns how many launches were bracketed (it may exceed capacity;
 * only the first `capacity` are recorded).  When `info` is not NULL, the
 * four values info[4k .. 4k+3] describe what launch k covered:
 *   NS classes (GRAM, POLY, APPLY, NS, NS_SMALL): the smaller and the larger
 *     side of the units (unpadded), the number of units, the tile size; an
 *     NS launch that also runs a single-unit pass (AUTO) carries that
 *     pass's smaller side, larger side and unit count in bits 32-63 of the
 *     first three values (zero otherwise), its own in bits 0-31;
 *   MOMENTUM: elements, algorithmic bytes (gradient or NS input read,
 *     momentum read and written, look-ahead written), units, 0;
 *   NORMALIZE: units, 0, 0, 0.
 * Events and the info array are owned by the caller. */
typedef struct {
  hipEvent_t* events;
  int64_t* info;     /* NULL, or 4 * capacity values */
  int32_t capacity;
  int32_t kind;
  int32_t count;
  int32_t reserved;
} muon_trace;

/* muon_step_batched / muon_newton_schulz_batched with an optional trace
 * (NULL = untraced, identical to the plain entry points). */
int muon_step_batched_traced(float* const* params, const void* const* grads,
                             float* const* momenta, const muon_matrix_desc* mats, int64_t n_mats,
                             const muon_hyper* h, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, muon_trace* trace);
int muon_newton_schulz_batched_traced(const float* const* x_in, float* const* o_out,
                                      const muon_matrix_desc* mats, int64_t n_mats,
                                      const muon_hyper* h, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream,
                                      muon_trace* trace);

/* Waits for `stream`, then reports whether any call on this workspace since
 * the previous muon_workspace_status (or since the workspace's first call)
 * had an NS launch stop early (a persistent one, or small units split on
 * chip, whose workgroups wait on each other): MUON_OK, or MUON_ERR_SCHEDULE, after
 * which the outputs of the calls in question are undefined.  The report is
 * sticky across calls and cleared by this function, so one check after a
 * series of steps covers all of them.  The step entry points return before
 * their kernels run and cannot see a stop: callers that need to know call
 * this function (the Python binding does with check=True).  Uses the first
 * 256 bytes of the workspace.  Errors: MUON_ERR_NULL, MUON_ERR_WORKSPACE
 * (fewer than 256 bytes), MUON_ERR_ALIGN, MUON_ERR_HIP. */
int muon_workspace_status(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* muon_status_string(int status);

/* ABI version of this header: 6. */
int muon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H_ */
