/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon optimizer step.
 *
 * One call performs, for every 2-D weight in a list, the Muon step the speedrun
 * pages describe:
 *
 *   m'  = beta * m + g                      momentum, no dampening
 *   u   = g + beta * m'  (Nesterov)  or  m'
 *   X0  = u / (||u||_F + eps),  transposed when rows > cols
 *   ns_steps x { A = X X^T ; B = b A + c A A ; X = a X + B X }
 *   O   = X (transposed back)
 *   W'  = W * (1 - lr * wd) - lr * sqrt(max(1, rows/cols)) * O
 *
 * Sources: "14 -- modded-nanogpt: the Speedrun Community", section 3 "Muon"
 * (pseudocode: momentum form, update sign, 5 iterations); "NanoGPT Speedrun"
 * (modded-nanogpt README mirror), Muon section (the Newton-Schulz routine:
 * eps = 1e-7 on the Frobenius norm, the transpose rule, coefficients
 * (3.4445, -4.7750, 2.0315); the practices list: Nesterov momentum, bfloat16
 * execution); same README, GPT-2 medium track ("standard weight decay").
 * Readings where the pages are silent: the Nesterov form u = g + beta m', the
 * decoupled lr-coupled decay on the old W, and the shape scale.
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major: element (i, j) at ptr[i * ld + j]; ld counts
 *     elements and must be >= cols.
 *   - Every data pointer is a device pointer on the handle's device, owned by
 *     the caller, and must stay valid until the stream has passed the work.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising (except the first call of a new
 *     signature, which waits for its plan upload).  The handle's workspaces
 *     are shared by its calls: calls on one handle must be ordered on one
 *     stream (or externally).
 *   - Validation happens before anything is enqueued; a call that returns an
 *     error enqueued nothing and changed no caller memory.
 *   - NaN/Inf inputs are not checked; they propagate within their matrix.
 *   - A handle is bound to one device and is not thread-safe; distinct handles
 *     are independent.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 6

typedef enum muon_status {
    MUON_OK = 0,
    MUON_ERR_INVALID_ARG = 1,  /* null pointer, bad size/ld, aliasing, bad ns_steps */
    MUON_ERR_DTYPE = 2,        /* unknown storage dtype or compute mode */
    MUON_ERR_NO_DEVICE = 3,    /* no HIP device, or the handle's device is gone */
    MUON_ERR_OOM = 4,          /* workspace allocation failed */
    MUON_ERR_HIP = 5           /* a HIP runtime call or launch failed; see muon_last_error */
} muon_status;

typedef enum muon_dtype {
    MUON_BF16 = 0,             /* bfloat16 storage */
    MUON_F32 = 1               /* float32 storage */
} muon_dtype;

typedef enum muon_compute {
    MUON_COMPUTE_BF16 = 0,     /* bf16 MFMA operands, fp32 accumulation; X kept between iterations
                                  to ~16 bits (bf16 copy + 8-bit remainder), A and B in bf16.
                                  Matrices (or blocks) with min(rows, cols) <= 64 run the iteration
                                  in fp32 in this mode too: their products cost next to nothing and
                                  bf16 operands cost them the most accuracy */
    MUON_COMPUTE_FP32 = 1      /* fp32 MFMA operands and storage: validation mode */
} muon_compute;

/* init flags */
#define MUON_INIT_PROFILE     0x1u   /* time kernel launches with HIP events (all roles, or see below) */
#define MUON_INIT_FAIL_ALLOC  0x2u   /* test hook: every workspace allocation fails (MUON_ERR_OOM) */
#define MUON_INIT_DEBUG       0x4u   /* debug checks: a guard band of a fixed pattern after every workspace
                                        buffer of muon_step's plans, checked after every step (which then
                                        waits for its stream); an overwritten band fails the call with
                                        MUON_ERR_HIP and the count of damaged words in muon_last_error */

/* Kernel roles, as named in muon_kernel_stats.name. */
typedef enum muon_role {
    MUON_ROLE_MOMENTUM = 0,    /* "momentum_norm" */
    MUON_ROLE_FINALIZE = 1,    /* "norm_finalize" */
    MUON_ROLE_GRAM = 2,        /* "ns_gram" */
    MUON_ROLE_POLY = 3,        /* "ns_poly" */
    MUON_ROLE_AXPY = 4,        /* "ns_axpy" (every iteration but the last) */
    MUON_ROLE_AXPY_UPDATE = 5, /* "ns_axpy_update" (last iteration and the weight update) */
    MUON_ROLE_DIRECT = 6,      /* "direct_update" (ns_steps == 0) */
    MUON_ROLE_FILL = 7,        /* "fill_zero" (workspace initialisation) */
    MUON_ROLE_ADAMW = 8,       /* "adamw" */
    MUON_ROLE_RESCALE = 9      /* "norm_rescale" (operand copy of inputs with an extreme norm) */
} muon_role;

/* With MUON_INIT_PROFILE, time only the roles whose bits are set in `mask`
 * (bit r = role r); no bits = every role.  Each timed launch carries its own
 * start/stop events, which costs a little time per launch. */
#define MUON_INIT_PROFILE_ROLES(mask) ((((uint32_t)(mask)) & 0x3FFu) << 16)

/* One weight matrix of the list handed to muon_step. */
typedef struct muon_matrix {
    void       *param;         /* rows x cols, `dtype`, updated in place */
    const void *grad;          /* rows x cols, `dtype`, read only */
    float      *momentum;      /* rows x cols float32, updated in place (start at 0) */
    float      *update_out;    /* optional rows x cols float32: receives O (validation); may be NULL */
    int64_t     rows, cols;    /* stored shape, both >= 1 */
    int64_t     ld_param, ld_grad, ld_mom, ld_update;   /* leading dims, elements, >= cols */
    int32_t     dtype;         /* muon_dtype of param and grad */
    int32_t     block_rows;    /* sub-block orthogonalisation: the matrix is cut into   */
    int32_t     block_cols;    /* block_rows x block_cols blocks (0 = the whole dimension;
                                  each must divide its dimension), and every block is a
                                  matrix of its own for the norm, the transpose rule, the
                                  iteration and the shape scale, as when query and key
                                  weights are orthogonalised in pairs of heads ("NanoGPT
                                  Speedrun", record list).  Momentum is elementwise and
                                  unaffected.  0, 0 = the plain step. */
    int32_t     reserved;      /* must be 0 */
} muon_matrix;

/* Hyperparameters, shared by every matrix of one call. */
typedef struct muon_hparams {
    float   lr;                /* learning rate */
    float   beta;              /* momentum, 0.95 on the pages */
    float   weight_decay;      /* decoupled: W *= 1 - lr * weight_decay */
    float   eps;               /* added to the Frobenius norm, 1e-7 on the pages */
    float   a, b, c;           /* quintic coefficients, (3.4445, -4.7750, 2.0315); finite, a != 0 */
    int32_t nesterov;          /* 0 or 1 */
    int32_t ns_steps;          /* 0..64; 5 on the pages */
    int32_t compute;           /* muon_compute */
    const float *coeffs;       /* optional host array of ns_steps triples (a_k, b_k, c_k), iteration k
                                  using the k-th in place of (a, b, c): per-iteration schedules such as
                                  Polar Express, named in the record list of "NanoGPT Speedrun"
                                  (modded-nanogpt README mirror); each finite, a_k != 0.  Read during
                                  the call only.  NULL = (a, b, c) for every iteration. */
} muon_hparams;

typedef struct muon_handle muon_handle;

/* Per-kernel launch statistics gathered when the handle was created with MUON_INIT_PROFILE. */
typedef struct muon_kernel_stats {
    char    name[48];          /* kernel role: "momentum_norm", "ns_gram", ... */
    int64_t launches;          /* completed launches timed */
    double  total_ms;          /* summed HIP-event durations */
} muon_kernel_stats;

/* One tensor of the list handed to muon_adamw_step: any parameter Muon does not
 * take (embeddings, output head, norm gains, biases), as `numel` contiguous
 * elements. */
typedef struct muon_adamw_tensor {
    void       *param;         /* numel elements, `dtype`, updated in place */
    const void *grad;          /* numel elements, `dtype`, read only */
    float      *exp_avg;       /* numel float32, first moment, updated in place (start at 0) */
    float      *exp_avg_sq;    /* numel float32, second moment, updated in place (start at 0) */
    int64_t     numel;         /* >= 0; 0 = nothing to do for this entry */
    int32_t     dtype;         /* muon_dtype of param and grad */
    int32_t     reserved;      /* must be 0 */
} muon_adamw_tensor;

/* AdamW hyperparameters, shared by every tensor of one call. */
typedef struct muon_adamw_hparams {
    float   lr;                /* learning rate, finite */
    float   beta1, beta2;      /* moment decays, each in [0, 1) */
    float   eps;               /* added to sqrt of the corrected second moment, finite, > 0 */
    float   weight_decay;      /* decoupled: p *= 1 - lr * weight_decay, finite */
    int32_t step;              /* 1-based step count t of this update (bias corrections 1 - beta^t) */
} muon_adamw_hparams;

/* Version of this header the library was built from (MUON_ABI_VERSION). */
int muon_abi_version(void);

/* Create a handle on HIP device `device`.  *out receives the handle (NULL on error).
 * Errors: MUON_ERR_INVALID_ARG (out == NULL, device out of range, unknown flag or role bits),
 * MUON_ERR_NO_DEVICE (no HIP device visible). */
muon_status muon_init(muon_handle **out, int device, uint32_t flags);

/* One Muon step over `n_mats` matrices (all steps above), enqueued on `stream`.
 *
 * Plans.  The first call for a given signature (the list of shapes, blocks,
 * dtypes, update_out presence and compute mode) builds a plan: tile lists,
 * device tables and a workspace of about 7 bytes per weight element in bf16
 * mode plus two min(rows,cols)^2 bf16 squares per matrix, zero-filled, then
 * waits for the stream once.  The handle keeps the plan of every signature it
 * has seen until muon_destroy (grow only): a later call with a known signature
 * allocates nothing and never synchronises, whichever signature came between.
 * Per plan the handle keeps up to 16 device copies of descriptor tables (the
 * call's pointers); a call whose pointers match a resident table enqueues
 * kernel launches only, otherwise it first uploads its table (an
 * asynchronous copy from pinned host memory) over the least recently used one.
 *
 * Graph capture.  A call on a stream that is being captured into a HIP graph
 * must find both its plan and a descriptor table with exactly its pointers
 * resident, i.e. the same call must have run once outside capture; otherwise
 * it returns MUON_ERR_INVALID_ARG and enqueues nothing.  The graph then reads
 * that plan's workspace and that table, which stay allocated and unchanged
 * until muon_destroy (a captured table is never overwritten; later calls with
 * other pointers use other tables).  Replays therefore act on the captured
 * buffers; they share the plan's workspace with eager calls of the same
 * signature, so replays and such calls must be ordered on one stream like any
 * two calls on the handle.  Destroying the handle invalidates the graph.
 *
 * A matrix cut into blocks (block_rows/block_cols) enters the plan as one entry
 * per block, in row-major block order; at most 65536 entries per call.
 * Normalisation is safe at any finite scale: the sum of squares runs in
 * double, and an input whose norm lies outside [2^-30, 2^30] is rescaled by a
 * power of two before the first products (one extra pass over its operand
 * copy; role MUON_ROLE_RESCALE, whose launch returns at once otherwise).
 * n_mats == 0 is a no-op.  Errors: MUON_ERR_INVALID_ARG (null handle/mats/hp with
 * n_mats > 0, null param/grad/momentum, rows or cols < 1, ld < cols, param == grad,
 * momentum aliasing param or grad, ns_steps outside 0..64, a == 0 or a non-finite
 * coefficient, also in coeffs, a block size < 0 or not dividing its dimension,
 * more than 65536 entries, reserved != 0, n_mats < 0, a capturing stream without
 * the resident plan and table described above), MUON_ERR_DTYPE, MUON_ERR_OOM,
 * MUON_ERR_HIP. */
muon_status muon_step(muon_handle *h, const muon_matrix *mats, int32_t n_mats,
                      const muon_hparams *hp, void *stream);

/* muon_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same step, with the same arguments, validation, errors and results
 * (bitwise) as muon_step, but every buffer it needs beyond the caller's
 * tensors (workspace, tile lists, units, norm partials, descriptor table)
 * lives in a static device array of 256 MiB per GPU (MUON_STATIC_SCRATCH_BYTES)
 * that the library reserves when it is loaded and holds until the process
 * ends.  Nothing is allocated: no hipMalloc/hipFree, no pinned host memory,
 * no events (profiling handles are not timed here).
 *   - A call whose workspace and tables exceed the scratch returns
 *     MUON_ERR_INVALID_ARG naming both sizes and enqueues nothing (roughly: up
 *     to ~30 M weight elements per call in bf16 mode).
 *   - Every call on a GPU shares that GPU's scratch, which keeps the last
 *     call's contents.  A call whose signature differs from the previous call's
 *     on the device clears the workspace (a fill kernel) and writes its tile
 *     lists; one whose pointers differ writes its descriptor table; either
 *     waits for `stream` before returning (the copies read host memory).  A
 *     call with the previous call's shapes and pointers enqueues kernels only.
 *   - Calls that overlap on one GPU (other streams, other threads, other
 *     handles) race on the scratch: order them.
 *   - The handle is used for its device and error text only; its plans are
 *     neither used nor created. */
#define MUON_STATIC_SCRATCH_BYTES (256u << 20)
muon_status muon_step_noalloc(muon_handle *h, const muon_matrix *mats, int32_t n_mats,
                              const muon_hparams *hp, void *stream);

/* Newton-Schulz only: out = NS(in) for one rows x cols matrix (normalise,
 * transpose rule, hp->ns_steps iterations with hp->a/b/c and hp->eps, in
 * hp->compute precision).  `in` has dtype `in_dtype` and leading dim ld_in;
 * `out` is rows x cols float32 with leading dim ld_out.  beta, lr, weight_decay
 * and nesterov are ignored.  Same errors as muon_step. */
muon_status muon_orthogonalize(muon_handle *h, const void *in, float *out,
                               int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out,
                               int32_t in_dtype, const muon_hparams *hp, void *stream);

/* One AdamW step over `n` tensors, enqueued on `stream`: for every element
 *
 *   m' = beta1 m + (1 - beta1) g ;  v' = beta2 v + (1 - beta2) g^2
 *   p' = p (1 - lr wd) - lr (m' / (1 - beta1^t)) / (sqrt(v' / (1 - beta2^t)) + eps)
 *
 * in float32 arithmetic (param rounded once to its dtype).  This is the update
 * the hybrid setup runs on the parameters Muon does not take ("14 --
 * modded-nanogpt", section 3; the Muon page, "Where Muon does not apply"); the
 * pages give no formula, so it is the standard AdamW (Loshchilov and Hutter,
 * decoupled weight decay, bias-corrected Adam moments).  One launch covers the
 * whole list.  The first call for a list of sizes/dtypes builds a plan (a few
 * bytes of device tables per 4096 elements); plans and descriptor tables are
 * cached and captured exactly as for muon_step.  n == 0 is a no-op.  Errors: MUON_ERR_INVALID_ARG (null
 * handle/tensors/hp with n > 0, a null buffer with numel > 0, numel < 0,
 * buffers of one tensor aliasing each other, beta outside [0, 1), eps <= 0,
 * a non-finite lr/eps/weight_decay, step < 1, reserved != 0, n < 0, a capturing
 * stream without the resident plan and table), MUON_ERR_DTYPE, MUON_ERR_OOM,
 * MUON_ERR_HIP. */
muon_status muon_adamw_step(muon_handle *h, const muon_adamw_tensor *tensors, int32_t n,
                            const muon_adamw_hparams *hp, void *stream);

/* Frobenius norms ||u||_F of the orthogonalised inputs of the most recent
 * muon_step (as enqueued: read after that step's kernels), one per plan entry (a blocked matrix has one per block, row-major)
 * in list order, copied to host memory `out` (n entries; the call
 * synchronises the stream).  Validation hook. */
muon_status muon_read_norms(muon_handle *h, float *out, int32_t n, void *stream);

/* Statistics per kernel role (profiling handles only); returns the number of
 * entries written (<= max), after waiting for the timed launches to finish. */
int32_t muon_kernel_stats_read(muon_handle *h, muon_kernel_stats *out, int32_t max);
void muon_kernel_stats_reset(muon_handle *h);

/* Workspace bytes currently held by the handle: the sum over the plans of
 * every signature seen (the plans' small device tables not included). */
int64_t muon_workspace_bytes(const muon_handle *h);

/* Free the handle and its workspace (waits for the device).  NULL is a no-op. */
muon_status muon_destroy(muon_handle *h);

/* Static text for a status code. */
const char *muon_status_str(muon_status s);

/* Text of the last error on this handle ("" if none); valid until the next call. */
const char *muon_last_error(const muon_handle *h);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */
