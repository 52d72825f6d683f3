/*
 * qz.h -- C ABI of libqz, a Hessian-weighted layer-wise weight quantizer for
 * AMD Instinct MI355X (gfx950).
 *
 * The library solves, for one linear layer with pretrained weights W_hat
 * [d_o x d_i] (row-major, one row per output channel) and calibration
 * activations X [n x d_i],
 *
 *     min_W  1/2 Tr((W - W_hat) H (W - W_hat)^T)   s.t. W on a b-bit grid,
 *     H = X^T X + lambda I,
 *
 * ("ADMM-Q: An Improved Hessian-based Weight Quantizer for Post-Training
 * Quantization of Large Language Models", technical summary, 1. problem
 * formulation; the pages store W as d_i x d_o, this ABI stores the transpose,
 * which leaves the objective unchanged) with two solvers: GPTQ ("061 · GPTQ"
 * tutorial, section 3, Algorithm 1) and ADMM-Q (ADMM-Q summary, 2. key
 * algorithmic components).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All array arguments are DEVICE pointers unless the comment says "host".
 *   The caller owns every buffer; the library never frees caller memory and
 *   allocates no device memory of its own: work buffers come from the caller
 *   through `ws`/`ws_bytes`, sized by the matching *_workspace() query and
 *   256-byte aligned (as hipMalloc returns them); a smaller or misaligned
 *   buffer gives QZ_EWORKSPACE.  Other arrays need only their element type's
 *   alignment (vector paths check and fall back to element access).
 *   Library-owned resources are per host thread and device and created on
 *   first use: four streams for GPTQ (two side streams of the factorisation,
 *   one for the grid fit beside it, one the factorisation's HIP graph is
 *   recorded on), that graph (kept while the call's arguments repeat), and a
 *   rocBLAS handle for the eigen-solver (which works in the caller's
 *   workspace).
 * - Matrices are dense row-major with the leading dimension equal to the
 *   column count, unless an ld argument is given.
 * - Arguments are checked before anything is enqueued; on a non-OK return the
 *   outputs are unspecified.
 * - Work is enqueued on `stream` (0 = the default stream).  Calls return after
 *   enqueueing unless marked SYNC; a SYNC call waits for its own work on
 *   `stream` and reports device-side failures (non-positive-definite H,
 *   non-finite data) through its status.
 * - Results are deterministic: no floating-point atomics are used, so two
 *   calls on the same inputs give the same bytes.
 * - qz_last_error() returns a thread-local message for the last non-OK status
 *   returned on the calling thread.
 */
#ifndef QZ_H
#define QZ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QZ_ABI_VERSION 2

typedef enum {
  QZ_OK = 0,
  QZ_EINVAL = -1,       /* bad argument (null pointer, size, bits, group, ...) */
  QZ_ENOTPD = -2,       /* H is not positive definite (add damping)            */
  QZ_ENONFINITE = -3,   /* NaN or Inf in H, W_hat or the ADMM iterates          */
  QZ_EHIP = -4,         /* a HIP runtime call failed                             */
  QZ_ESOLVER = -5,      /* the eigen-solver library failed                      */
  QZ_EWORKSPACE = -6    /* workspace too small                                   */
} qz_status;

typedef enum { QZ_BF16 = 0, QZ_F32 = 1 } qz_dtype;

/* ------------------------------------------------------------------ grid --
 * Per (row, group of `group_size` consecutive input columns) asymmetric grid:
 * value(c) = s * (c - z), c in {0 .. 2^bits - 1}, s fp32, z u8.
 * Fit rule (the pages give none; this is the library's reading): over the
 * group, lo = min(min v, 0), hi = max(max v, 0) (an all-zero group uses
 * [-1, 1]); s = fl32(fl32(hi - lo) / (2^b - 1)); z = clamp(rint(fl32(-lo/s)),
 * 0, 2^b - 1).  Codes: c = clamp(rint(fl32(x / s)) + z, 0, 2^b - 1), rint =
 * round half to even, IEEE fp32 division.  Scales and zeros are [d_o x d_i/g]
 * row-major.                                                                  */
#define QZ_GRID_CALLER 0x1u   /* scales/zeros are inputs, not fit from W_hat */

typedef struct {
  uint32_t struct_size;   /* sizeof(qz_grid) */
  int32_t bits;           /* 2 .. 8 */
  int32_t group_size;     /* >= 1, divides d_i; group_size == d_i is per output channel */
  uint32_t flags;         /* QZ_GRID_CALLER */
} qz_grid;

/* ---------------------------------------------------------------- Hessian --
 * qz_build_hessian: H = X^T X + lambda I with lambda = damp * mean(diag(X^T X))
 * (ADMM-Q summary, 1. problem formulation; damping: GPTQ tutorial, section 2,
 * "why damping is needed when calibration channels are collinear"), plus
 * diag(H) and Sigma = diag(H)^(-1/2) (ADMM-Q summary, 2., diagonal scaling),
 * and optionally the scaled Hessian Sigma H Sigma (unit diagonal).
 *
 *   X       [n x d_i], dtype xt (QZ_BF16: bf16 bit patterns; QZ_F32), n >= 1.
 *   flags   QZ_H_ACCUMULATE: add this call's X^T X to the unfinalised sum
 *             already in H (from a call made with QZ_H_NO_FINALIZE), so long
 *             calibration sets can be fed in token chunks;
 *           QZ_H_NO_FINALIZE: leave the raw sum X^T X in the UPPER triangle of
 *             H (lower triangle unspecified), no damping, diag/sigma/lambda
 *             untouched.
 *           Without QZ_H_NO_FINALIZE the call finishes H: mirrors it to a full
 *           symmetric matrix, adds lambda I and writes diag, sigma, lambda.
 *   H       [d_i x d_i] fp32 output (in/out with QZ_H_ACCUMULATE).
 *   diag, sigma  [d_i] fp32 outputs (nullable); lambda_out: 1 fp32 (nullable).
 *   H_scaled [d_i x d_i] fp32 output (nullable; not with QZ_H_NO_FINALIZE, must not
 *             alias H): H_ij sigma_i sigma_j in fp32 with the sigma above.
 *   ws      qz_hessian_workspace(n, d_i, xt) bytes (split-K partials, staging).
 * Products of bf16 values are exact in fp32; sums are fp32 (matrix cores); the
 * split sums are added in a fixed order.  Asynchronous.  Non-finite X gives
 * non-finite H, which qz_gptq and qz_admmq_prepare report as QZ_ENONFINITE.  */
#define QZ_H_ACCUMULATE 0x1u
#define QZ_H_NO_FINALIZE 0x2u

size_t qz_hessian_workspace(int64_t n, int64_t d_i, int32_t xt);
int qz_build_hessian(const void* X, int32_t xt, int64_t n, int64_t d_i, float damp,
                     uint32_t flags, float* H, float* diag, float* sigma, float* H_scaled,
                     float* lambda_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------------------- RTN --
 * qz_rtn: round-to-nearest of every weight on its own (ADMM-Q summary, problem
 * statement), on the grid fit from W (or the caller's grid with
 * QZ_GRID_CALLER).  Bit-exact with the fp32 definition above.
 *   W [d_o x d_i] (dtype wt); codes [d_o x d_i] u8 out; scales/zeros
 *   [d_o x d_i/g] out (in with QZ_GRID_CALLER).
 *   ws: qz_rtn_workspace(d_o, d_i) bytes (the call's status word), 256-byte
 *   aligned; calls on different streams need different workspaces.
 *   SYNC (reports non-finite W as QZ_ENONFINITE).                            */
size_t qz_rtn_workspace(int64_t d_o, int64_t d_i);
int qz_rtn(const void* W, int32_t wt, int64_t d_o, int64_t d_i, const qz_grid* grid,
           uint8_t* codes, float* scales, uint8_t* zeros, void* ws, size_t ws_bytes,
           hipStream_t stream);

/* qz_rtn_noalloc: qz_rtn for callers that cannot allocate device memory or hand over a
 * workspace (code under stream capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and errors as qz_rtn, without ws: the status
 * word lives in a 256-byte array of static device memory that the library holds on
 * each GPU it runs on until the process ends; the call allocates nothing.  The status
 * word is the only scratch, so every size qz_rtn accepts fits.  All calls on one GPU
 * share that word: calls that overlap on one GPU (other streams or threads) race on
 * it, and one may miss or misreport the other's non-finite weight.  SYNC.        */
int qz_rtn_noalloc(const void* W, int32_t wt, int64_t d_o, int64_t d_i, const qz_grid* grid,
                   uint8_t* codes, float* scales, uint8_t* zeros, hipStream_t stream);

/* ------------------------------------------------------------------- GPTQ --
 * qz_gptq: GPTQ tutorial, section 3 (Algorithm 1).  R is the upper Cholesky
 * factor of H^{-1} (H already damped by qz_build_hessian; no damping is added
 * here).  Columns are processed in blocks of B in a common order for all rows
 * (`perm`, or natural order); in each block every column is rounded on its
 * row's static grid, E = (w - q) / R_jj is kept and the block's remaining
 * columns get E R[j, j:b]; the later columns get the matrix-core product update
 * W[:, b:] -= E R[a:b, b:], applied lazily in two levels (a block's E updates the
 * rest of its group of up to 512 columns at once, the group's E all later columns
 * after the group: the same sums in a different order).
 *   H      [d_i x d_i] fp32 symmetric positive definite.
 *   W_hat  [d_o x d_i] (dtype wt).
 *   B      block size, 1 .. 128.
 *   perm   [d_i] int32 processing order (a permutation of 0..d_i-1) or NULL.
 *          Groups are always contiguous ranges of the ORIGINAL columns, and
 *          codes are written in original column positions.
 *   codes  [d_o x d_i] u8 out; scales/zeros [d_o x d_i/g] out (in with
 *          QZ_GRID_CALLER).
 * R is computed in fp64 (blocked Cholesky of the reversed H, triangular
 * inverse) and used in fp32; the factorisation runs part of its work on two
 * library-owned side streams (default priority, one pair per host thread and
 * device) that join `stream` before the call goes on, so the call still orders
 * on `stream` only.  The factorisation's operations are recorded once into a
 * HIP graph and replayed with one launch on `stream` while H, perm, the
 * workspace and the sizes are the same pointers and values as in the previous
 * call on this host thread and device (the graph reads the buffers' current
 * contents); a `stream` that is being captured gets the operations directly.  SYNC: the codes and the grid are complete when the call
 * returns; QZ_ENOTPD when a pivot of the factorisation is <= 1e-12 of its
 * diagonal entry (or not finite), QZ_ENONFINITE for non-finite H or W_hat.   */
size_t qz_gptq_workspace(int64_t d_o, int64_t d_i, int32_t B);
int qz_gptq(const float* H, const void* W_hat, int32_t wt, int64_t d_o, int64_t d_i,
            const qz_grid* grid, int32_t B, const int32_t* perm,
            uint8_t* codes, float* scales, uint8_t* zeros,
            void* ws, size_t ws_bytes, hipStream_t stream);

/* qz_gptq_noclip: qz_gptq without clipping (Babai page, technical summary, 2.3 and
 * 3: the error bound of Theorem 5 holds when codes may take any integer value).  The
 * code of a column is rint(w / s) + z unclamped (kept inside the int32 range), so the
 * stored grid is the same but codes [d_o x d_i] are int32 and may leave [0, 2^b - 1].
 * Arguments, workspace (qz_gptq_workspace), sync and errors as qz_gptq.          */
int qz_gptq_noclip(const float* H, const void* W_hat, int32_t wt, int64_t d_o, int64_t d_i,
                   const qz_grid* grid, int32_t B, const int32_t* perm,
                   int32_t* codes, float* scales, uint8_t* zeros,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------- orders and error bound --
 * Babai page, technical summary, 2.3: without clipping the error of a row is
 * bounded by a quarter of its squared scales weighted by the diagonal D of the
 * LDL factorisation of the reordered Hessian (Theorem 5); the bound depends on the
 * order; the min-pivot order (the smallest remaining diagonal at every LDL step)
 * keeps the trace of D small and act order (descending diagonal) approximates it.
 * Orders are quantization orders for qz_gptq's perm: perm[j] = the original column
 * quantized j-th.  The LDL elimination runs in the reverse of the quantization
 * order (the column quantized last is eliminated first).
 *
 * qz_order:
 *   kind QZ_ORDER_ACT: columns by descending H_jj, ties to the smaller index.
 *   kind QZ_ORDER_MIN_PIVOT: the reverse of the elimination order of a pivoted LDL
 *     of H in fp64 that takes the smallest Schur-complement diagonal at every step
 *     (among equal pivots the larger original index is eliminated first, so ties go
 *     to the smaller index in quantization order, as in act order).  H must be
 *     symmetric (the pivoted factorisation reads rows of the trailing matrix).
 *   H [d_i x d_i] fp32; perm [d_i] int32 out.
 *   pivots (device, nullable, MIN_PIVOT only): [d_i] fp64 out, the LDL pivot of the
 *     column quantized j-th (the D of Theorem 5 for that order).
 *   ws: qz_order_workspace(d_i, kind) bytes, 256-byte aligned (8 d_i^2 bytes for
 *     MIN_PIVOT).  SYNC: QZ_ENONFINITE for a non-finite H, QZ_ENOTPD when a pivot
 *     is <= 1e-12 of its column's diagonal.
 *
 * qz_error_bound: per row the Theorem 5 bound on the layer objective of
 *   qz_objective without clipping, in quantization order perm (NULL = natural):
 *     row_bound[r] = 1/8 sum_j D_j s(r, perm[j])^2
 *   (the 1/4 of Theorem 5 times f's 1/2), D_j = the LDL pivot of the column quantized
 *   j-th = 1 / R_jj^2 of qz_gptq's factor for that order (fp64 Cholesky of the
 *   reversed, reordered H).  scales [d_o x d_i/group_size] (the grid the codes are
 *   on).  row_bound (device, nullable) [d_o] fp64 out; out_host (host, nullable):
 *   the sum over rows.  ws: qz_error_bound_workspace(d_o, d_i) bytes, 256-byte
 *   aligned.  SYNC: QZ_EINVAL for a perm that is not a permutation, QZ_ENOTPD,
 *   QZ_ENONFINITE as qz_gptq.                                                 */
#define QZ_ORDER_ACT 1
#define QZ_ORDER_MIN_PIVOT 2
size_t qz_order_workspace(int64_t d_i, int32_t kind);
int qz_order(const float* H, int64_t d_i, int32_t kind, int32_t* perm, double* pivots,
             void* ws, size_t ws_bytes, hipStream_t stream);
size_t qz_error_bound_workspace(int64_t d_o, int64_t d_i);
int qz_error_bound(const float* H, int64_t d_i, const int32_t* perm, const float* scales,
                   int64_t d_o, int32_t group_size, double* row_bound, double* out_host,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------- ADMM-Q --
 * qz_admmq_prepare: Sigma = diag(H)^(-1/2), H~ = Sigma H Sigma and its
 * eigendecomposition H~ = V diag(Lambda) V^T (ADMM-Q summary, 2.: the
 * W-update is evaluated through an eigendecomposition of the Hessian).  The
 * decomposition runs in fp64 in the rocSOLVER library (a library call standing
 * in for host LAPACK); V and Lambda are returned in fp32.
 *   H [d_i x d_i] fp32; V [d_i x d_i] fp32 out, V[j][k] = component j of
 *   eigenvector k; Lambda [d_i] ascending; sigma [d_i].
 *   ws: qz_admmq_prepare_workspace(d_i) bytes, 256-byte aligned: the fp64 copy of
 *   H~ (8 d_i^2 bytes), the eigenvalue and off-diagonal vectors and the solver
 *   library's scratch (its size is asked of the library, so the query needs the
 *   device current; it returns 0 on failure).  d_i <= 46340.
 *   SYNC: QZ_ENONFINITE for a non-finite H or a non-positive diagonal entry,
 *   QZ_ESOLVER when the solver fails or does not converge.                    */
size_t qz_admmq_prepare_workspace(int64_t d_i);
int qz_admmq_prepare(const float* H, int64_t d_i, float* V, float* Lambda, float* sigma,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* qz_admmq: the ADMM-Q splitting loop in scaled coordinates W~ = W Sigma^{-1}:
 *   for t = t0 .. t0+iters-1, rho_t = rho0 * gamma^t (ADMM-Q summary, 2.,
 *   convergence under the penalty schedule):
 *     M  = D~ - U
 *     W~ = ((P + rho_t M V) diag(1/(Lambda + rho_t))) V^T, P = W~_hat V Lambda
 *          (two fp32 matrix-core products)                         [W-update]
 *     if refresh_every > 0 and t % refresh_every == 0: refit each group's grid
 *          from min/max of the continuous iterate W~ Sigma, clamped into the
 *          group's initial range [lo_0, hi_0]                  [grid refresh]
 *     C  = codes of (W~ + U) Sigma, D~ = s (C - z) Sigma^{-1}      [D-update]
 *     U  = (U + W~ - D~) * rho_t / rho_{t+1}                    [dual update]
 *     residuals[t - t0] = (||W~ - D~||_F, rho_t ||D~ - D~_prev||_F)
 *   Start (without QZ_ADMM_WARM_START): t0 = 0, the static grid fit from W_hat
 *   (or the caller's with QZ_GRID_CALLER), C = RTN(W_hat), U = 0.
 *   With QZ_ADMM_WARM_START the state (codes, scales, zeros, U) is read from
 *   the output buffers and the loop resumes at p->t0.
 *   Output: the last discrete iterate (codes) and its grid.
 *   V, Lambda, sigma from qz_admmq_prepare.  U [d_o x d_i] fp32 in/out
 *   (nullable unless WARM_START).  residuals [iters x 2] fp32 (nullable).
 *   SYNC: QZ_ENONFINITE if W_hat is not finite or a residual became NaN.    */
#define QZ_ADMM_WARM_START 0x1u
#define QZ_ADMM_REFRESH_UNCLAMPED 0x2u  /* refit without the [lo_0, hi_0] clamp */
#define QZ_ADMM_REFRESH_FROM_Z 0x4u     /* refit from (W~ + U) Sigma            */
#define QZ_ADMM_DUAL_NO_RESCALE 0x8u    /* U = U + W~ - D~ (no rho_t/rho_{t+1}) */

typedef struct {
  uint32_t struct_size;   /* sizeof(qz_admm) */
  int32_t iters;          /* >= 0 */
  float rho0;             /* > 0 */
  float gamma;            /* > 0 */
  int32_t refresh_every;  /* 0 = never */
  uint32_t flags;
  int32_t t0;             /* first iteration index with QZ_ADMM_WARM_START */
} qz_admm;

size_t qz_admmq_workspace(int64_t d_o, int64_t d_i, int32_t group_size, int32_t iters);
int qz_admmq(const float* V, const float* Lambda, const float* sigma,
             const void* W_hat, int32_t wt, int64_t d_o, int64_t d_i,
             const qz_grid* grid, const qz_admm* params,
             uint8_t* codes, float* scales, uint8_t* zeros, float* U, float* residuals,
             void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- packing --
 * Storage format (the ADMM-Q summary says the output keeps GPTQ's format; the
 * bit layout is this library's reading): each row is a little-endian stream
 * of 32-bit words, code i in bits [i*bits, (i+1)*bits), least significant bit
 * first (codes may straddle words), zero-padded to ceil(cols*bits/32) words.
 *   codes [rows x cols] u8 (every code < 2^bits); out [rows x words] u32.
 * Asynchronous.                                                             */
int64_t qz_packed_words(int64_t cols, int32_t bits);
int qz_pack(const uint8_t* codes, int64_t rows, int64_t cols, int32_t bits, uint32_t* out,
            hipStream_t stream);
int qz_unpack(const uint32_t* in, int64_t rows, int64_t cols, int32_t bits, uint8_t* codes,
              hipStream_t stream);

/* -------------------------------------------------------------- objective --
 * The layer objective both solvers minimise (ADMM-Q summary, methodology, 1.
 * problem formulation; GPTQ tutorial, section 2, the curvature-weighted cost):
 *   f = 1/2 sum_r (q_r - w_r)^T H (q_r - w_r),   q = s (C - z) per (row, group),
 * with w_r the rows of W_hat.  Computed as D = Q - W_hat (fp32), the product D H
 * on the matrix cores with each output element multiplied by D in the same pass
 * (D H is never stored), row sums in fp64 in a fixed order.
 *   H [d_i x d_i] fp32 symmetric; W_hat [d_o x d_i] (dtype wt); codes [d_o x d_i];
 *   scales, zeros [d_o x d_i/group_size].
 *   row_f (device, nullable): [d_o] fp64 per-row objectives.
 *   out_host (host, nullable): f.  When given the call is SYNC and reports a
 *   non-finite weight or scale as QZ_ENONFINITE; otherwise it is asynchronous.
 *   ws: qz_objective_workspace(d_o, d_i) bytes, 256-byte aligned.            */
size_t qz_objective_workspace(int64_t d_o, int64_t d_i);
int qz_objective(const float* H, const void* W_hat, int32_t wt, const uint8_t* codes,
                 const float* scales, const uint8_t* zeros, int64_t d_o, int64_t d_i,
                 int32_t group_size, double* row_f, double* out_host, void* ws,
                 size_t ws_bytes, hipStream_t stream);
/* qz_objective_i32: the same objective for int32 codes (qz_gptq_noclip's output);
 * same workspace, sync and errors.                                            */
int qz_objective_i32(const float* H, const void* W_hat, int32_t wt, const int32_t* codes,
                     const float* scales, const uint8_t* zeros, int64_t d_o, int64_t d_i,
                     int32_t group_size, double* row_f, double* out_host, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------- local search --
 * Pairwise-swap local search after a solver (ADMM-Q summary, methodology, 2. key
 * algorithmic components, the local-search item: discrete moves that swap values
 * between positions of an output channel, evaluated by their direct effect on the
 * reconstruction error, in parallel).  The grid (scales, zeros) stays fixed.  Moves
 * are defined inside one group: one code +-1, or two codes j < k changed by a, b in
 * {-1, +1}.  The gradient (Q - W_hat) H is formed once on the matrix cores (fp32) and
 * kept up to date with the accepted moves.  Each step: every (row, group) proposes its
 * move with the smallest exact change of the objective (qz_objective's f) if negative,
 * ties to the smallest (j, k, a, b); each row accepts proposals in ascending group
 * order while the change plus the exact interaction with the moves it already accepted
 * stays negative, then applies them, so f never rises.  A row stops after a step that
 * accepts none of its proposals; rows are independent.
 *   grid: bits and group_size (at most 128 columns; it divides d_i); scales, zeros
 *   [d_o x d_i/group_size] are inputs.  codes [d_o x d_i] u8 in/out.
 *   max_steps >= 0; the search stops after a step that accepts no move.
 *   moves_host (host, nullable): [max_steps] moves accepted per step (entries past
 *   the last step run are not written); steps_host (host, nullable): steps that
 *   accepted at least one move.  SYNC (every step reads the move count).
 *   ws: qz_local_search_workspace(d_o, d_i, group_size) bytes, 256-byte aligned.  */
size_t qz_local_search_workspace(int64_t d_o, int64_t d_i, int32_t group_size);
int qz_local_search(const float* H, const void* W_hat, int32_t wt, int64_t d_o, int64_t d_i,
                    const qz_grid* grid, const float* scales, const uint8_t* zeros,
                    uint8_t* codes, int32_t max_steps, int32_t* moves_host,
                    int32_t* steps_host, void* ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------- timing --
 * Per-kernel timing for measurement tools: while enabled, the library records a
 * HIP event pair around each of its kernel launches, on the stream the kernel
 * runs on, and qz_timing_read sums the elapsed times per kernel kind.
 *   qz_timing_enable(1) starts recording (calling process, any device); 0 stops.
 *   qz_timing_read fills launches[k] and total_ms[k] for k < min(max_kinds,
 *   QZ_TIMING_KINDS) (host arrays, may be NULL), waits for the recorded events
 *   (SYNC), then, if reset != 0, drops the records.  Returns the number of kinds.
 *   qz_timing_kind_name(k) names kind k ("" when out of range).              */
#define QZ_TIMING_KINDS 16
int qz_timing_enable(int on);
int qz_timing_read(int64_t* launches, double* total_ms, int max_kinds, int reset);
const char* qz_timing_kind_name(int kind);

/* ---------------------------------------------------------------- misc ---- */
const char* qz_last_error(void);
int qz_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QZ_H */
