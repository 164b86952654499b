/*
 * profk.h: C ABI of the MI355X (gfx950) Prof-K exact top-k library.
 *
 * The method is "Prof-K: Probabilistic One-Pass Filtering for Efficient
 * Top-k Selection" (arXiv HTML page, cited below as P1; its earlier version
 * on the bittide mirror is P2).  A uniform sample of S indices sets a
 * threshold tau at the t-th largest sampled entry; one streaming pass keeps
 * every entry at or above tau in a candidate buffer of capacity M and counts
 * them exactly (R); an exact selection on the buffer gives the top k.  When
 * the run-time check k <= R <= M fails the sample is redrawn; after the last
 * attempt an exact full-tensor selection runs.  The result is always the
 * exact top-k (P1 abstract, §3 stage 4).
 *
 * Order and ties.  The pages assume distinct entries (P1 §4 "Notation and
 * Conventions").  This library uses the total order "larger value first,
 * then lower index"; -0.0 and +0.0 compare equal; every NaN ranks above
 * +inf and NaNs tie with each other (broken by index).  Outputs are sorted
 * in that order; out_vals[j] is a bit copy of x[out_idx[j]].
 *
 * Memory.  Every x / out pointer is a DEVICE pointer owned by the caller.
 * The library owns a workspace per (device, stream), sized O(S + M + k)
 * (never O(N)), grown on demand and freed by profk_release().  Pointers to
 * option / parameter / stats structs are HOST pointers.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Work is enqueued on it.  The host waits once per attempt for the
 * count R and the check k <= R <= M (P1 App. D "Cost of the Run-Time Check"),
 * which the device publishes into pinned host memory; profk_topk /
 * profk_topk_ex then return while the last kernel, which sorts and writes the
 * outputs, may still run.  The outputs are complete in stream order: any later
 * work on the same stream (or after synchronising it) sees them.  The batched,
 * stage and fallback paths synchronise the stream before returning.
 *
 * Errors.  Every entry point returns a status code; nothing throws across
 * the ABI.  profk_strerror() gives a message (HIP errors include the HIP
 * error string of the failing call, kept per thread).
 *
 * Limits.  Indices are 32-bit inside the keys.  profk_topk / profk_topk_ex
 * take N >= 2^32 (up to about 2^38) by cutting x into segments of fewer than
 * 2^32 values and merging their exact top-k lists (P1 App. D, Table 4);
 * profk_topk_approx, the batched form, the stage entry points and
 * profk_solve return PROFK_EUNSUPPORTED for N >= 2^32 per row.
 */
#ifndef PROFK_H
#define PROFK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PROFK_OK 0
#define PROFK_EINVAL (-1)       /* bad argument (null pointer, k < 1, k > N, eps outside (0,1), ld < N ...) */
#define PROFK_EUNSUPPORTED (-2) /* N >= 2^32 per row where not supported (see Limits) */
#define PROFK_ENOMEM (-3)       /* workspace allocation failed */
#define PROFK_EHIP (-4)         /* a HIP runtime call failed */
#define PROFK_EINTERNAL (-5)    /* a device-side consistency check failed */
#define PROFK_ESCRATCH (-6)     /* profk_topk_approx_noalloc: the call needs more than the static scratch */

/* Overrides for tests and experiments.  Zero-initialise for defaults. */
typedef struct profk_options {
  int64_t s_override;     /* > 0: use this sample size S instead of the rule */
  int64_t s_min;          /* 0: 32768 (P2 §4 "Optimal Sample Size") */
  int64_t s_max;          /* 0: 131072 (same place) */
  double s_prefactor;     /* <= 0: 1.0; c in S*_raw = c (k (N-k))^(1/3) */
  int64_t force_t;        /* > 0: threshold rank t instead of Theorem 4's t* */
  int64_t force_M;        /* > 0: buffer capacity M (>= k) instead of M* */
  int32_t max_attempts;   /* < 0 or unset (0 with use_max_attempts = 0): 6 (P1 §3 stage 4) */
  int32_t use_max_attempts; /* nonzero: max_attempts is taken as given (0 = straight to the exact path) */
  int32_t force_fallback; /* nonzero: skip the sampled attempts, run the exact full selection */
  int32_t timing;         /* nonzero: time the filter kernel with HIP events (stats.filter_ms) */
  int32_t param_mode;     /* PROFK_PARAMS_EXACT (0): Theorem 4's (t*, M*), memoised (P1 §4 Eq. 7);
                             PROFK_PARAMS_FAST: the closed-form surrogates of P1 Algorithm 1 (Eq. 10-12),
                             elementary arithmetic only, computed on every call and not memoised */
  int32_t s_rule;         /* PROFK_S_RULE_CUBE_ROOT (0): S = c (k (N-k))^(1/3) clamped to [s_min, s_max]
                             (P2 Theorem 5); PROFK_S_RULE_COST_MODEL: P1 Algorithm 1 lines 1-4 (the cost
                             model of Proposition 7 with the calibrated ratio r(k); defaults s_min = 2^14,
                             s_max = 2^18); PROFK_S_RULE_MI355X: the same lines with the cost ratio
                             measured on MI355X (one constant 1/r = 0.022 for every k, no floor for
                             k/N > 2^-10; defaults s_min = 2^12, s_max = 2^17) */
  double cost_a, cost_b;  /* PROFK_S_RULE_COST_MODEL: 1/r(k) = cost_a log2(k) - cost_b for k > 2^7 (P1 App.
                             E.1); both <= 0: the page's calibration, 0.594 and 4.29 */
  int64_t refine_wait_ticks; /* exact mode, k > 64: bound on the refinement's one wait for all of its
                             workgroups, in ticks of the device's 100 MHz clock (0: 25,000,000,
                             i.e. 0.25 s); a wait that runs out sends the attempt to the multi-pass
                             refinement (same result).  < 0: the wait counts as run out at once
                             (a hook for tests of that path) */
} profk_options;

#define PROFK_PARAMS_EXACT 0
#define PROFK_PARAMS_FAST 1
#define PROFK_S_RULE_CUBE_ROOT 0
#define PROFK_S_RULE_COST_MODEL 1
#define PROFK_S_RULE_MI355X 2

/* The parameter choice for one (N, k, eps) (P1 §4 Theorem 4; P2 §4). */
typedef struct profk_params {
  int64_t N, k;
  double eps;
  double eps_a, eps_b; /* budget split eps/2 + eps/2 */
  double z_a;          /* Phi^-1(1 - eps_a) */
  double z;            /* z_A + z_B (P2 Algorithm 1) */
  double S_raw;        /* c (k (N-k))^(1/3) before the clamp */
  int64_t S;           /* sample size used */
  int64_t t_star;      /* P1 Eq. 7 (-1 in PROFK_PARAMS_FAST mode: not computed) */
  int64_t M_star;      /* P1 Eq. 7 (-1 in PROFK_PARAMS_FAST mode) */
  double M_cf;         /* P2 Corollary 4, Eq. 12 */
  int64_t t_eq6;       /* P2 Eq. 6 (reported only) */
  int64_t t, M;        /* operating pair: t = t*, M = max(M*, ceil(M_cf)) unless forced; in
                          PROFK_PARAMS_FAST mode the Algorithm 1 pair (t, M) */
  double p_recall;     /* Pr(R < k) at (t, M), P1 Eq. 5 (-1 in PROFK_PARAMS_FAST mode: not computed) */
  double p_overflow;   /* Pr(R > M) at (t, M), P1 Eq. 6 (-1 in PROFK_PARAMS_FAST mode) */
  double E_R, Var_R;   /* P2 Lemma 1, Eq. 2 */
  int32_t direct_exact; /* 1: sampling cannot pay off here; the call runs the exact full selection */
  int32_t reserved;
} profk_params;

#define PROFK_STATS_ATTEMPTS 8
typedef struct profk_stats {
  int32_t attempts;       /* sampled attempts made */
  int32_t fallback;       /* 1: the exact full selection produced the output */
  int64_t S, t, M;        /* operating parameters */
  int64_t R[PROFK_STATS_ATTEMPTS];         /* exact filter count per attempt (row 0 when batched) */
  int32_t fail_mode[PROFK_STATS_ATTEMPTS]; /* 0 ok, 1 R < k, 2 R > M */
  uint64_t workspace_bytes; /* bytes of device workspace held for this (device, stream) */
  double filter_ms;       /* filter kernel time of the last attempt (options.timing) */
  int64_t rows_retried;   /* batched: rows that needed more than one attempt */
  int64_t rows_fallback;  /* batched: rows finished by the exact full selection */
  int64_t refine_multipass; /* attempts whose refinement needed the multi-pass radix select
                               (a value bin too large for one workgroup: ties, narrow ranges) */
  int64_t segments;       /* N >= 2^32: segments the input was cut into (0 otherwise); the
                             fields above are then segment 0's, except attempts (the most of
                             any segment), fallback (any), refine_multipass and filter_ms
                             (summed over segments) */
} profk_stats;

/*
 * profk_topk: exact top-k of one flat fp32 tensor x[0..N) (P1 §3, Algorithm
 * "The Prof-K Algorithm", stages 1-4, with the retry of stage 4).
 *   x        device, N floats, any alignment
 *   N        1 <= N; N >= 2^32 takes the segmented path (see Limits)
 *   k        1 <= k <= N
 *   eps      failure budget per attempt, 0 < eps < 1 (P1 §4 Theorem 4)
 *   seed     64-bit seed of the sampler's Philox stream; attempt a uses
 *            counter space a.  The output does not depend on it.
 *   out_vals device, k floats; out_idx device, k int64 (sorted, see top)
 */
int profk_topk(const float* x, int64_t N, int64_t k, double eps, uint64_t seed, float* out_vals,
               int64_t* out_idx, void* stream);

/* profk_topk with overrides (opt may be NULL) and statistics (st may be NULL). */
int profk_topk_ex(const float* x, int64_t N, int64_t k, double eps, uint64_t seed, float* out_vals,
                  int64_t* out_idx, void* stream, const profk_options* opt, profk_stats* st);

/*
 * Approximate mode (P1 App. D "Cost of the Run-Time Check"; App. E.2): one
 * sampled attempt with no host read of the count.  Every step is enqueued on
 * `stream` and the call returns without waiting, so it can be captured in a
 * HIP graph once a first call has sized the workspace (a call that must grow
 * the workspace allocates and is not capturable).  The output is the exact
 * top-k of the candidates the attempt kept: it is the exact top-k whenever
 * k <= R <= M held, which fails with probability at most eps.  The outcome of
 * the check is written, in stream order, to *info (device memory).
 *   info     device pointer to one profk_approx_info, or NULL
 *   other arguments as profk_topk_ex (opt may be NULL; max_attempts and
 *   timing are ignored)
 */
typedef struct profk_approx_info {
  int64_t R;          /* exact filter count of the attempt (N when the exact selection ran) */
  int64_t M;          /* buffer capacity of the attempt */
  int32_t status;     /* 0: k <= R <= M held, the output is the exact top-k;
                         1: R < k: positions R..k-1 hold index -1 and value -inf;
                         2: R > M: the output is the top-k of the M kept candidates */
  int32_t exact_path; /* 1: the configuration went to the exact full selection (status 0) */
} profk_approx_info;

int profk_topk_approx(const float* x, int64_t N, int64_t k, double eps, uint64_t seed, float* out_vals,
                      int64_t* out_idx, profk_approx_info* info, void* stream, const profk_options* opt);

/*
 * profk_topk_approx_noalloc: profk_topk_approx for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It calls no hipMalloc,
 * hipFree, hipHostMalloc or other allocating runtime routine; its workspace is
 * a static device array of PROFK_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds from the time the library is loaded until the process
 * ends.  The first call on a device looks up the array's device address
 * (hipGetSymbolAddress): make that call outside graph capture.  The first call
 * for a (N, k, eps, options) configuration computes and memoises its
 * parameters on the host (host heap only).
 *   Arguments, outputs and *info are those of profk_topk_approx; the results
 *   are bit-identical to profk_topk_approx's for the same arguments.
 *   Returns PROFK_ESCRATCH, without enqueuing anything, when the configuration
 *   needs more workspace than the array holds (64 MiB: every k up to 2^19 at
 *   N up to 2^30 under every S rule; larger k or N may not fit).
 * Every call on one GPU uses that GPU's single array, which keeps what the last
 * call left in it; each call first clears the parts that must start at zero.
 * Calls that overlap in time on one GPU (other streams, other threads) race on
 * the array and give wrong results: serialise them.
 */
#define PROFK_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

int profk_topk_approx_noalloc(const float* x, int64_t N, int64_t k, double eps, uint64_t seed, float* out_vals,
                              int64_t* out_idx, profk_approx_info* info, void* stream, const profk_options* opt);

/*
 * profk_topk_batched: row-wise exact top-k of B rows (P1 §3: the procedure
 * is applied to each batch element; App. C: per-row threshold, buffer and
 * counter).  Row r is x[r*ld_x .. r*ld_x + N).  The budget is split eps/B
 * per row so that the whole call meets eps (P1 App. E.2).  Only the rows
 * that fail the check are redrawn.
 *   out_vals device B*k floats, out_idx device B*k int64 column indices in [0, N)
 */
int profk_topk_batched(const float* x, int64_t B, int64_t N, int64_t ld_x, int64_t k, double eps,
                       uint64_t seed, float* out_vals, int64_t* out_idx, void* stream);

int profk_topk_batched_ex(const float* x, int64_t B, int64_t N, int64_t ld_x, int64_t k, double eps,
                          uint64_t seed, float* out_vals, int64_t* out_idx, void* stream,
                          const profk_options* opt, profk_stats* st);

/*
 * profk_topk_batched_approx: the batched form in approximate mode (P1 App. E.2,
 * "Batched Inputs" and Table 6: approximate mode on batches, the budget split
 * eps/B per row; App. D: no run-time check).  One sampled attempt per row, every
 * step enqueued on `stream`, no host wait: the call returns at once and, once a
 * first call has sized the workspace, can be captured in a HIP graph.  Row r's
 * output is the exact top-k of the candidates its attempt kept, which is its
 * exact top-k whenever k <= R <= M held for it (probability at least
 * 1 - eps/B); the outcome goes to info[r] as in profk_topk_approx (status 1:
 * positions R..k-1 hold index -1 and value -inf; status 2: the top-k of the M
 * kept).  Rows short enough that the sample would not pay off are sorted whole
 * (exact, exact_path = 1).  Shapes outside the batched kernels (k > 16384) run
 * profk_topk_approx row by row, still stream-ordered.
 *   info     device pointer to B profk_approx_info records (required)
 *   other arguments as profk_topk_batched_ex (opt may be NULL; max_attempts,
 *   force_fallback and timing are ignored)
 */
int profk_topk_batched_approx(const float* x, int64_t B, int64_t N, int64_t ld_x, int64_t k, double eps,
                              uint64_t seed, float* out_vals, int64_t* out_idx, profk_approx_info* info, void* stream,
                              const profk_options* opt);

/*
 * profk_solve: host-only parameter choice (P1 §4 Theorem 4 / Eq. 5-7; the
 * S rule and closed forms of P2 §4 Theorem 5, Corollary 4, Algorithm 1).
 * Memoised per (N, k, eps, options) (P1 §4 "Fast Approximate Parameter
 * Computation": parameters are cached per configuration).  With
 * opt->param_mode = PROFK_PARAMS_FAST the pair (t, M) comes from the closed
 * forms of P1 Algorithm 1 instead, in a few microseconds, without the memo.
 * No GPU needed.
 */
int profk_solve(int64_t N, int64_t k, double eps, const profk_options* opt, profk_params* out);

/*
 * Stage entry points: each runs one stage of the hot path on the GPU, for
 * inspection and parity tests.  All array pointers are device pointers.
 *
 * profk_stage_sample: stage 1 (P1 §3): the S distinct indices of the
 *   sample of (seed, attempt), in unspecified order, into out_idx[0..S).
 *   1 <= S <= N/2.
 */
int profk_stage_sample(const float* x, int64_t N, int64_t S, uint64_t seed, int32_t attempt,
                       int64_t* out_idx, void* stream);

/*
 * profk_stage_threshold: stages 1-2 (P1 §3): tau = the t-th entry, in the
 *   total order, of the sample of (seed, attempt).  out_tau_val (1 float),
 *   out_tau_idx (1 int64).  1 <= t <= S <= N/2.
 */
int profk_stage_threshold(const float* x, int64_t N, int64_t S, int64_t t, uint64_t seed,
                          int32_t attempt, float* out_tau_val, int64_t* out_tau_idx, void* stream);

/*
 * profk_stage_batched_sample: stages 1-2 of the batched form (P1 §3: the
 *   procedure applied to each batch element; App. C: a threshold per row) for
 *   rows 0..B-1 of x (row r at x + r*ld_x, N values).  Row r's sample is drawn
 *   from the counter space of (seed, attempt, row r), exactly as in
 *   profk_topk_batched.  Outputs (device):
 *     out_idx      B*S int64: row r's S distinct sampled indices (in [0, N), in
 *                  unspecified order) at out_idx[r*S .. r*S+S)
 *     out_tau_val  B floats, out_tau_idx B int64: tau_r = the t-th entry of row
 *                  r's sample in the total order (index within the row)
 *   1 <= t <= S, 2S <= N, ld_x >= N, B <= 65535.  Rows of up to 2^20 values use
 *   the per-row bitmap sampler (then S <= 2^17), longer rows the grid sampler,
 *   as profk_topk_batched does.  Synchronises the stream.  A device-side
 *   inconsistency in any row gives PROFK_EINTERNAL.
 */
int profk_stage_batched_sample(const float* x, int64_t B, int64_t N, int64_t ld_x, int64_t S, int64_t t,
                               uint64_t seed, int32_t attempt, int64_t* out_idx, float* out_tau_val,
                               int64_t* out_tau_idx, void* stream);

/*
 * profk_stage_filter: stage 3 (P1 §3; App. C "The Filter Kernel"): with the
 *   given tau = (tau_val, tau_idx), out_R[0] = R = number of entries at or
 *   before tau in the total order (exact, even past capacity), and the
 *   indices of min(R, M) of them in out_cand_idx[0..min(R,M)) (unspecified
 *   order; which ones are kept on overflow is unspecified).
 */
int profk_stage_filter(const float* x, int64_t N, float tau_val, int64_t tau_idx, int64_t M,
                       int64_t* out_cand_idx, int64_t* out_R, void* stream);

/*
 * profk_read_ceiling: measurement helper, not part of the selection.  Reads
 *   x[0..N) once with the filter's loads (dwordx4, non-temporal; stage 3 of P1
 *   §3 reads every value once, App. C) and nothing else, and XORs the XOR of
 *   all N values' bit patterns into *out_fold (device, one uint64).  Its
 *   time on the same buffer is the practical ceiling of the filter's one-read
 *   roofline on the device at hand.  x must be 16-byte aligned;
 *   blocks_per_cu in 0..16 (0: 2) sets the persistent grid (256 threads per
 *   block).  Enqueued on `stream`; does not wait.
 */
int profk_read_ceiling(const float* x, int64_t N, int32_t blocks_per_cu, uint64_t* out_fold, void* stream);

/* Message for a status code (thread-local detail for PROFK_EHIP). */
const char* profk_strerror(int code);

/* Frees every cached workspace (all devices and streams).  Not thread-safe
 * against concurrent calls. */
void profk_release(void);

#ifdef __cplusplus
}
#endif

#endif /* PROFK_H */
