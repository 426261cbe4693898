/*
 * shampoo.h -- C-ABI of libshampoo_mi355x.so: the Shampoo optimizer step on
 * one AMD Instinct MI355X (gfx950).
 *
 * Method: "Scalable Second Order Optimization for Deep Learning" (Anil, Gupta,
 * Koren, Regan, Singer).  The pages describe it in the Shampoo-at-scale
 * podcast transcript: a 2-D weight keeps one statistics matrix per dimension,
 * L (rows) and R (columns) (cues 6-7); each step adds three pieces of work --
 * accumulate gradient outer products into L and R, take the inverse fourth
 * roots of L and R, and multiply the gradient by them (cue 10); the roots are
 * expensive, computed by coupled Newton iteration, in double precision when
 * the statistics are ill-conditioned (cue 12), and only every so often, the
 * last ones being reused in between (cue 14); over-large layers are split into
 * blocks that are preconditioned separately (Lemma 2, cue 16).  The paper runs
 * the roots on host CPUs; this library runs the whole step on the GPU.
 *
 * Not on the pages, and fixed by this library's configuration instead:
 * exponential moving average of the statistics (beta2), damping
 * eps = eps_rel * lambda_max of each factor, per-block grafting of the update
 * magnitude to diagonal Adagrad, heavy-ball momentum (beta1), diagonal Adagrad
 * for tensors with a dimension above max_precond_dim and sparse-row Adagrad
 * for embedding tables.
 *
 * Conventions for every call below:
 *   - All device pointers are HIP device memory on the current device; all
 *     tensors are fp32, row-major, contiguous.
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).  Calls
 *     enqueue work and return without waiting, except shampoo_bind_state and
 *     shampoo_get_diagnostics, which wait for their own work.  Calls on one
 *     handle must be ordered (issue them on one stream).  A handle is not
 *     thread-safe.
 *   - Return value: SHAMPOO_OK (0) or a negative shampoo_status.  Argument and
 *     state errors are detected on the host before anything is enqueued.
 *     Numerical conditions (non-finite statistics, a root that failed) never
 *     fail a call: they are recorded per factor and read back with
 *     shampoo_get_diagnostics.  No C++ exception crosses this interface.
 */
#ifndef SHAMPOO_MI355X_H
#define SHAMPOO_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct shampoo_s shampoo_t; /* opaque; owns host memory only (the plan) */

typedef enum {
    SHAMPOO_OK = 0,
    SHAMPOO_E_ARG = -1,         /* null pointer, bad size or shape, bad config value  */
    SHAMPOO_E_STATE = -2,       /* no state bound, or state too small                 */
    SHAMPOO_E_HIP = -3,         /* a HIP call or kernel launch failed                 */
    SHAMPOO_E_NOMEM = -4,       /* host allocation failed                             */
    SHAMPOO_E_UNSUPPORTED = -5  /* valid but not supported (e.g. root_p not 1,2,4,8)  */
} shampoo_status;

typedef enum {
    SHAMPOO_ROOT_F32 = 0,  /* every factor's coupled-Newton root in fp32                  */
    SHAMPOO_ROOT_F64 = 1,  /* every factor in fp64                                         */
    SHAMPOO_ROOT_AUTO = 2  /* fp32 first; factors whose estimated condition number of
                              S + eps I exceeds fp64_cond_threshold are redone in fp64 */
} shampoo_root_mode;

typedef enum {
    SHAMPOO_DENSE = 0,       /* 2-D weight: Shampoo blocks, or diagonal Adagrad when a
                                dimension exceeds max_precond_dim                    */
    SHAMPOO_SPARSE_ROWS = 1  /* embedding table updated by sparse-row Adagrad        */
} shampoo_tensor_kind;

typedef struct {
    int64_t rows, cols;  /* shape of the weight (and of its gradient) */
    int32_t kind;        /* shampoo_tensor_kind */
    int32_t reserved;    /* must be 0 */
} shampoo_tensor_desc;

typedef struct {
    int32_t block_size;       /* b: Lemma-2 block edge; blocks are top-left aligned b x b
                                 tiles, the last row/column of blocks ragged (>= 1)      */
    int32_t max_precond_dim;  /* dense tensors with a dimension above this use diagonal
                                 Adagrad; 0 = no limit                                   */
    int32_t root_p;           /* p of the inverse p-th root; the pages use 4 (cue 10)    */
    int32_t newton_iters;     /* coupled-Newton iterations per root at p = 4 (e.g. 20);
                                 a factor with exponent p < 4 runs
                                 ceil(newton_iters log g_4 / log g_p), g_p = ((p+1)/p)^p
                                 (p = 2: 23, p = 1: 26 for 20), the steps that close the
                                 same eigenvalue gap                                     */
    int32_t root_mode;        /* shampoo_root_mode                                       */
    int32_t lanczos_steps;    /* Krylov steps for lambda_max; 0 = adaptive: stop at the
                                 first check (after 12 steps, every 4th to 32, every 8th
                                 after) where the top Ritz pair's residual is within
                                 5e-5 of theta, at most 64 steps; the kappa estimate
                                 uses min(8, this), 8 when 0                            */
    int32_t root_parts;       /* staggered root pass (cue 14-16: roots are computed off
                                 the critical path and swapped in): 0 or 1 = one pass
                                 over every factor; P >= 2 also plans P parts, part q
                                 holding the factors of the blocks b with b % P == q
                                 (shampoo_compute_inverse_roots_part, shampoo_step)      */
    int32_t large_layer;      /* dense tensors too large for Shampoo blocks (a dimension
                                 above max_precond_dim): 0 = diagonal Adagrad; 1 = when
                                 the other dimension fits, one-sided preconditioning of
                                 that side only (Lemma 1, cue 16: for a giant embedding
                                 or softmax layer only one of L or R is used), with the
                                 exponent -2/root_p so that the one factor carries the
                                 whole -1/2 of full-matrix Adagrad; needs an even root_p.
                                 With 1, sparse-row tables whose columns fit (any, when
                                 max_precond_dim is 0) get the column side instead of
                                 sparse-row Adagrad                                      */
    int32_t apply_precision;  /* the two products of D = P_L G P_R for blocks above 128
                                 (and D = G P_R of a one-sided column side): 0 = fp32
                                 matrix cores; 1 = split precision (bf16x3): each fp32
                                 operand x split into hi = bf16(x), lo = bf16(x - hi),
                                 the product formed as hi*hi + hi*lo + lo*hi on the bf16
                                 matrix cores with fp32 accumulation (about 2^-16
                                 relative per term instead of 2^-24), the Adagrad pass
                                 of those blocks fused into the first product; needs
                                 root_p >= 4 (the roots' condition kappa^(1/p) amplifies
                                 the rounding, p = 1 at kappa 1e6: ~1e-2 of the update)  */
    int32_t reserved;         /* must be 0                                                */
    double beta1;             /* momentum: mom <- beta1 mom + U                          */
    double beta2;             /* statistics: S <- beta2 S + (1-beta2) outer(G) (beta2<1),
                                 S <- S + outer(G) when beta2 == 1; 1 - beta2 is formed in
                                 double, so beta2 is double here                         */
    double lr;                /* W <- W - lr mom                                          */
    double eps_rel;           /* eps = eps_rel * lambda_max(S) per factor                */
    double graft_eps;         /* delta in A = G / (sqrt(a) + delta)                      */
    double fp64_cond_threshold; /* AUTO mode: kappa(S + eps I) above this -> fp64 root  */
    double newton_tol;        /* 0 = every root runs its full iteration count, the
                                 plain coupled iteration.  In (0, 1): the iteration stops
                                 once M_k is within newton_tol of I (its convergence
                                 test; near I the error squares each step), at most the
                                 full count.  An fp32 root of a factor up to 128 (fused
                                 kernel) stops one step after ||M_k - I||_F < newton_tol.
                                 The batched chains (fp32 above 128, every fp64 root)
                                 take scaled steps (M_k scaled by mu_k, X_k by
                                 mu_k^(1/p), mu_k chosen from a bound on the spectrum of
                                 M_k that the eps floor gives, the same for every factor)
                                 and run one step (fp32) or two (fp64) past the first
                                 step count at which that bound puts every eigenvalue
                                 of M_k within newton_tol of 1 (10 and 11 steps at
                                 p = 4, eps_rel 1e-6, newton_tol 1e-3); the last step
                                 forms X only.  With
                                 eps_rel = 0 there is no bound: the full count.  E.g. 1e-3 */
} shampoo_config;

/* Row-sparse gradient of one SHAMPOO_SPARSE_ROWS table: n_rows distinct row
 * ids (int32, device) and an n_rows x cols fp32 block of row gradients
 * (device).  Rows must be distinct within one call; order is free. */
typedef struct {
    const int32_t* rows;
    const float* row_grads;
    int64_t n_rows;
} shampoo_sparse_rows;

/* One factor's numbers from the last shampoo_compute_inverse_roots. */
typedef struct {
    double lambda_max;   /* Krylov estimate of the largest eigenvalue of S           */
    double eps;          /* eps_rel * lambda_max: the damping added to S              */
    double kappa_est;    /* estimate of kappa(S + eps I) from the fp32 root (0: none) */
    double residual;     /* max |M - I| of the committed coupled iteration's last M
                            (the batched chains form no M in their last step: M_{N-1}) */
    int32_t block;       /* block index (see shampoo_block_info)                      */
    int32_t side;        /* 0: L (rows), 1: R (columns)                               */
    int32_t dim;         /* factor dimension                                          */
    int32_t status;      /* bit mask of SHAMPOO_FACTOR_* below                         */
    int32_t iters;       /* coupled-Newton steps run (0: none, e.g. a zero factor)    */
    int32_t reserved;
} shampoo_factor_diag;

enum {
    SHAMPOO_FACTOR_NONFINITE_INPUT = 1,  /* S not finite: previous root kept            */
    SHAMPOO_FACTOR_NONFINITE_ROOT = 2,   /* iteration went non-finite: previous kept    */
    SHAMPOO_FACTOR_RESIDUAL_HIGH = 4,    /* committed, but max|M_N - I| > 1e-2          */
    SHAMPOO_FACTOR_FP64 = 8,             /* root computed in fp64                        */
    SHAMPOO_FACTOR_ZERO = 16             /* lambda_max <= 0 (no statistics): root = I   */
};

/* Where one block's state lives in the bound state buffer (byte offsets).
 * A one-sided block (large_layer = 1) is a whole tensor with a single factor:
 * the fields of the side that is not preconditioned are ld 0, factor -1 and
 * offsets -1; its statistic S is kept in both triangles and its roots are
 * (S + eps I)^(-2/root_p). */
typedef struct {
    int32_t tensor;       /* index into the tensor list                               */
    int32_t row0, col0;   /* top-left element of the block in the tensor               */
    int32_t rows, cols;   /* m_b, n_b (ragged at the edges)                            */
    int32_t ld_l, ld_r;   /* leading dimension (padded) of the L- and R-side matrices  */
    int32_t factor_l, factor_r; /* factor indices (diagnostics order)                 */
    int32_t one_sided;    /* 1: one-sided block of a large layer (Lemma 1)             */
    int64_t off_l, off_r;       /* fp64 statistics L (rows x rows), R (cols x cols),
                                   row-major with leading dims ld_l, ld_r; symmetric,
                                   only the upper triangle (column >= row) is kept    */
    int64_t off_pl, off_pr;     /* fp32 roots P_L, P_R                                */
    int64_t off_pl64, off_pr64; /* fp64 roots, or -1 when root_mode is F32             */
} shampoo_block_layout;

/*
 * shampoo_create -- build the plan for a list of tensors.
 * cfg: hyper-parameters (copied).  tensors: n_tensors descriptors (copied).
 * out: receives the handle.  Host only: no HIP call, no device memory.
 * Dense tensors whose dimensions are both <= max_precond_dim (or any, when it
 * is 0) are split into Lemma-2 blocks (cue 16); each block gets an L and an R
 * factor.  With large_layer = 1, a dense tensor with one dimension above
 * max_precond_dim and the other within it, and a sparse-row table whose
 * columns fit, become one more block each, numbered after every Lemma-2
 * block (tensors in order), with one factor for the side that fits (R for a
 * table).  Errors: SHAMPOO_E_ARG (null pointer, n_tensors < 1, a dimension
 * < 1, block_size < 1, newton_iters < 1, beta2 outside (0,1], eps_rel < 0,
 * unknown kind or root_mode, large_layer or apply_precision not 0 or 1,
 * reserved not 0), SHAMPOO_E_UNSUPPORTED (root_p not in {1,2,4,8}; root_p odd
 * with large_layer = 1; apply_precision 1 with root_p < 4; a factor
 * dimension above 1024; rows above 2^31 - 1 or cols above 2^20),
 * SHAMPOO_E_NOMEM.
 * Scratch: the batched coupled-Newton iteration (fp32 factors above 128 and
 * every fp64 root) runs in chunks of factors whose scratch (six ld x ld
 * matrices per factor) stays within 4 GiB per precision; the environment
 * variable SHAMPOO_NEWTON_SCRATCH_BYTES, read here, sets another limit (a
 * chunk holds at least one factor).  In AUTO mode the fp64 chain runs on the
 * factors routed to fp64 only, packed in factor order into the leading chunks
 * of their class.
 */
int shampoo_create(const shampoo_config* cfg, int32_t n_tensors,
                   const shampoo_tensor_desc* tensors, shampoo_t** out);

/* Bytes of device state the handle needs (statistics, roots, Adagrad and
 * momentum accumulators, scratch).  The caller allocates it (e.g. a PyTorch
 * uint8 tensor), 256-byte aligned, and keeps it alive and in place for the
 * handle's life.  Host only. */
int shampoo_state_bytes(const shampoo_t* h, size_t* bytes);

/* Attach the caller's device state buffer and initialise it on `stream`:
 * statistics, accumulators and momentum zero, roots the identity, and the
 * plan's descriptor tables uploaded.  Waits for that work to finish.
 * Errors: SHAMPOO_E_ARG (null, not 256-byte aligned), SHAMPOO_E_STATE (bytes
 * below shampoo_state_bytes), SHAMPOO_E_HIP. */
int shampoo_bind_state(shampoo_t* h, void* dev_state, size_t bytes, void* stream);

/* Statistics (cue 10): for every block, L <- beta2 L + w G_b G_b^T and
 * R <- beta2 R + w G_b^T G_b, w = 1 - beta2 (1 when beta2 == 1): fp32
 * gradients, fp64 products and accumulation on MFMA, fp64 storage.  A
 * one-sided block updates only its one factor, S <- beta2 S + w G^T G (R) or
 * w G G^T (L), the product split over the long dimension and the partial
 * products summed in a fixed order.  A sparse-row table with one-sided
 * preconditioning adds the products of this call's row gradients,
 * S <- beta2 S + w g^T g (only decaying when it lists no rows).  grads:
 * n_tensors device pointers, read only; entries of tensors without blocks
 * are ignored (may be NULL).  sparse: as in shampoo_precondition_and_apply;
 * read only for sparse-row tables with one-sided preconditioning, may be NULL
 * when the plan has none.  Errors: SHAMPOO_E_ARG, SHAMPOO_E_STATE,
 * SHAMPOO_E_HIP. */
int shampoo_update_stats(shampoo_t* h, const float* const* grads,
                         const shampoo_sparse_rows* sparse, void* stream);

/* Inverse roots (cue 10, 12, 14): for every factor S, lambda_max by Lanczos,
 * eps = eps_rel * lambda_max, then P = (S + eps I)^(-1/p) (p = root_p, or
 * root_p / 2 for the factor of a one-sided block) by coupled Newton
 * iteration (newton_iters steps, or fewer for a fused fp32 root that meets
 * newton_tol; fp32, fp64 or routed per root_mode).  A
 * factor with non-finite S or a non-finite result keeps its previous root; a
 * factor with lambda_max <= 0 gets P = I.  The caller decides the cadence
 * (call it when step % k == 0); in between, the last roots are used.
 * Errors: SHAMPOO_E_STATE, SHAMPOO_E_HIP. */
int shampoo_compute_inverse_roots(shampoo_t* h, void* stream);

/* One part of a staggered root pass: the inverse roots, exactly as
 * shampoo_compute_inverse_roots computes them, of the factors of the blocks b
 * with b % root_parts == part (block numbering: tensors in order, blocks
 * row-major within a tensor).  Calling part (t / (k/P)) % P whenever
 * t % (k/P) == 0 (P = root_parts dividing the cadence k) refreshes every root
 * once per k steps and spreads the cost of a pass evenly over the steps.
 * Errors: SHAMPOO_E_ARG (root_parts < 2 or part out of range),
 * SHAMPOO_E_STATE, SHAMPOO_E_HIP. */
int shampoo_compute_inverse_roots_part(shampoo_t* h, int32_t part, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * root pass as shampoo_compute_inverse_roots, every factor, whose batched
 * coupled-Newton iterates (factors above 128 in fp32, every fp64 root) live
 * in a static device array of the library, 64 MiB per GPU (held from the
 * first shampoo_bind_state on that GPU until the process ends), instead of
 * the scratch part of the state buffer; no split-K stages.  It calls no
 * hipMalloc, hipFree or other allocating routine, and records no profiling
 * events.  Results: statistics-derived diagnostics and routing as the whole
 * pass; roots to rounding of it (products summed without the split).  Every
 * call on one GPU shares that GPU's array and leaves its last contents there
 * (nothing in it needs clearing: each chunk writes every iterate it reads),
 * so calls that overlap on one GPU (several handles or streams at once) race.
 * Must be called with the device current at shampoo_bind_state.
 * Errors: SHAMPOO_E_STATE (not bound, a part in flight, another device
 * current), SHAMPOO_E_UNSUPPORTED (a chain slot larger than the array: not
 * for factors up to 1024), SHAMPOO_E_HIP. */
int shampoo_compute_inverse_roots_noalloc(shampoo_t* h, void* stream);

/* The same part computed in the background (cues 14-16: the roots are
 * produced off the critical path while training continues on the last ones,
 * and swapped in when ready).  shampoo_roots_async_begin enqueues on `stream`
 * a snapshot of the part's statistics and current roots, then runs the part's
 * root pass on a stream of the library's own (default priority) that reads
 * the snapshot and writes staged roots; the calls that follow on `stream`
 * (statistics, apply) keep using the current roots.  shampoo_roots_async_end
 * makes `stream` wait for that pass and swaps the staged roots in (a factor
 * whose root failed keeps its previous one); it does nothing when no part is
 * in flight.  The result does not depend on timing: roots computed from the
 * statistics after the step that began the part take effect where end is
 * called.  Only one part can be in flight; while one is, the synchronous root
 * calls fail with SHAMPOO_E_STATE and the part's diagnostics are being
 * written.  Errors: SHAMPOO_E_ARG (root_parts < 2 or part out of range),
 * SHAMPOO_E_STATE, SHAMPOO_E_HIP. */
int shampoo_roots_async_begin(shampoo_t* h, int32_t part, void* stream);
int shampoo_roots_async_end(shampoo_t* h, void* stream);

/* Preconditioned multiply and update (cue 10): for every block
 * D_b = P_L G_b P_R; a <- a + G*G; A = G / (sqrt(a) + graft_eps);
 * U_b = D_b ||A_b||_F / ||D_b||_F (0 when ||D_b|| = 0);
 * mom <- beta1 mom + U; W <- W - lr mom.  A one-sided block takes D = G P (R)
 * or P G (L) and grafts over the whole tensor; other tensors above
 * max_precond_dim take U = A.  A sparse-row table with one-sided
 * preconditioning takes, on its listed rows, a_r += g_r^2,
 * A = g / (sqrt(a) + graft_eps), D = g P_R, U = D ||A||_F / ||D||_F (norms over
 * the listed rows) and W_r -= lr U_r: no momentum, and rows not listed are
 * untouched; row ids outside the table are skipped by the accumulator and
 * weight updates (their gradients still enter the statistics).  Sparse tables: for each listed row r, a_r += g_r^2 and
 * W_r -= lr g_r / (sqrt(a_r) + graft_eps); other rows untouched; no momentum.
 * params: n_tensors device pointers, updated in place.  grads: as in
 * shampoo_update_stats (dense tensors must be non-NULL).  sparse: NULL when
 * there are no sparse tables, else n_tensors entries (entries of dense tensors
 * ignored; n_rows == 0 allowed).  Errors: SHAMPOO_E_ARG, SHAMPOO_E_STATE,
 * SHAMPOO_E_HIP. */
int shampoo_precondition_and_apply(shampoo_t* h, float* const* params,
                                   const float* const* grads,
                                   const shampoo_sparse_rows* sparse, void* stream);

/* Root selector of shampoo_step. */
enum {
    SHAMPOO_ROOTS_NONE = -1,  /* no roots this step                                      */
    SHAMPOO_ROOTS_ALL = -2    /* every root (shampoo_compute_inverse_roots); a value
                                 0 <= q < root_parts selects part q instead
                                 (shampoo_compute_inverse_roots_part)                    */
};

/* One optimizer step: shampoo_update_stats, then the roots that `roots`
 * selects, then shampoo_precondition_and_apply, with the same arguments.  On
 * a step without roots the statistics of a block (G, L, R) and its apply (G,
 * a, P, mom, W) share only read-only inputs, so every block of at most
 * 128 x 128 gets both from one kernel that reads G once, and (unless
 * per-kernel profiling is enabled) the statistics of the larger blocks run on
 * a stream of the library's (default priority) beside the apply: forked from `stream` by an event after this call's
 * pointer upload and joined back into it before the call's last work, so
 * work issued on `stream` afterwards sees the whole step (the fork and join
 * are events, which stream capture into a graph follows).  Results:
 * statistics and Adagrad accumulators bit for bit those of the separate
 * calls; momentum and weights to rounding (the two block norms of the graft
 * are summed in another fixed order).  Errors: as the separate calls, and
 * SHAMPOO_E_ARG for an invalid `roots`. */
int shampoo_step(shampoo_t* h, float* const* params, const float* const* grads,
                 const shampoo_sparse_rows* sparse, int32_t roots, void* stream);

/* Number of factors (2 per Lemma-2 block, 1 per one-sided block) and blocks
 * in the plan.  Host only. */
int shampoo_num_factors(const shampoo_t* h, int32_t* n_factors, int32_t* n_blocks);

/* Copy up to `cap` factor records from the last root pass into host memory
 * (`out`), in factor order.  Waits for `stream`.  Errors: SHAMPOO_E_ARG,
 * SHAMPOO_E_STATE, SHAMPOO_E_HIP. */
int shampoo_get_diagnostics(shampoo_t* h, shampoo_factor_diag* out, int32_t cap, void* stream);

/* Layout of block `block` (0 <= block < n_blocks).  Host only. */
int shampoo_block_info(const shampoo_t* h, int32_t block, shampoo_block_layout* out);

/* Byte offsets in the state buffer of tensor `tensor`'s Adagrad accumulator
 * and momentum (both fp32, the tensor's shape; mom_off = -1 for sparse
 * tables), and its block range [first_block, first_block + n_blocks).
 * Host only. */
int shampoo_tensor_info(const shampoo_t* h, int32_t tensor, int64_t* adagrad_off,
                        int64_t* mom_off, int32_t* first_block, int32_t* n_blocks);

/* Per-kernel GPU time, for measurement tools.  While enabled, every kernel
 * launch of the calls above is bracketed by two HIP events recorded on the
 * call's stream (a few microseconds of host time per launch, no device
 * synchronisation), and shampoo_step runs every stage in order on that
 * stream (no statistics beside the apply), so each launch is timed alone.  shampoo_profile_read waits for the recorded events, adds
 * their elapsed times per kernel family into `out` (up to `cap` records, in a
 * fixed order; *n_out receives the number written) and resets the counters.
 * Errors: SHAMPOO_E_ARG, SHAMPOO_E_HIP. */
typedef struct {
    char name[32];       /* kernel family, e.g. "newton_gemm_f32"                     */
    int64_t launches;    /* launches since the last read                              */
    double total_ms;     /* summed event-to-event GPU time of those launches          */
} shampoo_kernel_time;

int shampoo_profile_enable(shampoo_t* h, int32_t on);
int shampoo_profile_read(shampoo_t* h, shampoo_kernel_time* out, int32_t cap, int32_t* n_out);

/* Machine peaks measured on the current device, for measurement tools that
 * report kernel rates as fractions of a peak.  None of the method's
 * arithmetic: the matrix-core issue rate of the MFMA instructions the
 * products use (fp32 v_mfma_f32_32x32x2f32, fp64 v_mfma_f64_16x16x4f64, bf16
 * v_mfma_f32_32x32x16_bf16), every wave of a full grid issuing independent
 * products from registers with no memory traffic; and the best of a few
 * shapes of a plain device-to-device copy (bytes read plus bytes written, per
 * second).  Each figure is the median of three timed launches (HIP events on
 * `stream`) after one warm-up; the call waits for them. */
typedef struct {
    double mfma_f32_tflops;  /* TFLOP/s, 2 flops per multiply-add                  */
    double mfma_f64_tflops;
    double mfma_bf16_tflops; /* v_mfma_f32_32x32x16_bf16 (fp32 accumulation)         */
    double copy_gbs;         /* GB/s (1e9 bytes), read + write                       */
    int64_t copy_bytes;      /* bytes read by one copy (half the scratch, rounded)  */
} shampoo_peaks;

/* scratch: device memory, 256-byte aligned, at least 2 MiB; the copy reads
 * its first half and writes its second half, the MFMA probes write a few KiB
 * at its start (contents are overwritten, never interpreted).  Needs no
 * handle.  Errors: SHAMPOO_E_ARG (null, unaligned or too small scratch),
 * SHAMPOO_E_HIP. */
int shampoo_measure_peaks(shampoo_peaks* out, void* scratch, size_t scratch_bytes, void* stream);

/* Free the handle (host memory only; the caller frees the state buffer). */
void shampoo_destroy(shampoo_t* h);

/* Static text for a status code. */
const char* shampoo_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* SHAMPOO_MI355X_H */
