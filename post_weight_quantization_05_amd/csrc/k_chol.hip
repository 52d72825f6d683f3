// Inverse Cholesky factor for GPTQ: upper-triangular R with R^T R = H^{-1}
// (GPTQ tutorial, section 3: the algorithm runs on the upper Cholesky factor of the
// damped inverse curvature, chosen over repeated inverse updates for stability).
//
// Route (no explicit inverse of H): with J the reversal permutation, factor the
// reversed matrix J H J = L L^T (lower Cholesky); then H = (J L J)(J L J)^T with
// J L J upper triangular, so H^{-1} = ((J L J)^{-1})^T (J L J)^{-1} and
// R = (J L J)^{-1} = J L^{-1} J.  Both steps are blocked right-looking fp64 algorithms
// on 64 x 64 tiles:
//   Cholesky   -- per block column: factor + invert the diagonal block (one
//                 workgroup, in LDS), scale the panel below by the inverse, update
//                 the trailing lower triangle (tile GEMMs);
//   inverse    -- X = L^{-1} by block forward substitution, S <- I: per block row i,
//                 X[i, :i] = L_ii^{-1} S[i, :i], then S[r, :i] -= L[r, i] X[i, :i] for
//                 the rows below (tile GEMMs).
// The matrix is padded to a multiple of 64 with an identity block, which keeps every
// tile full.  A pivot <= 1e-12 of its original diagonal entry (or not finite) sets
// the not-positive-definite flag; the caller reads it at its sync point (the GPTQ
// tutorial's damping section: a failed factorisation means more damping is needed).
// Output: R^T (lower, row-major) in fp32, the layout the GPTQ kernels read.
#include <vector>

#include "qz_internal.h"

namespace qz {

namespace {

constexpr int NB = 64;
constexpr int kThreads = 256;

// A[i][j] = Hp[d-1-i][d-1-j] (Hp = H[perm][:, perm]) for i, j < d; identity padding.
__global__ __launch_bounds__(kThreads) void init_reversed(const float* __restrict__ H, int64_t d,
                                                          const int32_t* __restrict__ perm,
                                                          double* __restrict__ A, int64_t lda,
                                                          double* __restrict__ diag0,
                                                          uint32_t* __restrict__ flag) {
  const int64_t total = lda * lda;
  bool bad = false;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / lda, j = e % lda;
    double v;
    if (i < d && j < d) {
      int64_t si = d - 1 - i, sj = d - 1 - j;
      if (perm) { si = perm[si]; sj = perm[sj]; }
      const float h = H[si * d + sj];
      bad |= !__builtin_isfinite(h);
      v = static_cast<double>(h);
    } else {
      v = (i == j) ? 1.0 : 0.0;
    }
    A[e] = v;
    if (i == j) diag0[i] = v;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, FLAG_NONFINITE);
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), l);
  return __hiloint2double(hi, lo);
}

// 1 / sqrt(p) for p > 0: the hardware estimate refined by two Newton steps
// y <- y (3 - p y^2) / 2 (each step squares the relative error).
__device__ __forceinline__ double rsqrt_f64(double p) {
  double y = __builtin_amdgcn_rsq(p);
  y = y * (1.5 - 0.5 * p * y * y);
  y = y * (1.5 - 0.5 * p * y * y);
  return y;
}

// Factor diagonal block k in place (lower) and write its inverse to Dinv[k].
// One wavefront: lane i holds row i of the block in registers during the factorisation
// (all 64 loads of a row in flight at once).  Per column j the pivot is broadcast
// from lane j (readlane) and every lane forms its reciprocal square root; the new
// column goes to LDS twice, row-major (Ls, for the inverse) and column-major (Lc, so the
// rank-one update of the rows below reads one contiguous run of uniform broadcasts).
// The inverse is formed by forward substitution with lane i holding column i, each sum
// split over four independent partial sums.
__global__ __launch_bounds__(NB) void diag_block(double* __restrict__ A, int64_t lda, int64_t k,
                                                 const double* __restrict__ diag0,
                                                 double* __restrict__ Dinv,
                                                 uint32_t* __restrict__ flag) {
  __shared__ double Ls[NB][NB + 2];   // L row-major (even stride: 16-byte pair reads)
  __shared__ double Lc[NB][NB];       // Lc[j][l] = L[l][j]
  __shared__ double rinv[NB];
  const int i = threadIdx.x;
  const int64_t k0 = k * NB;
  double a[NB];
  const double* __restrict__ row = A + (k0 + i) * lda + k0;
#pragma unroll
  for (int c = 0; c < NB; ++c) a[c] = (c <= i) ? row[c] : 0.0;
  const double tol = 1e-12 * diag0[k0 + i];
  bool notpd = false;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const double p = readlane_f64(a[j], j);          // the pivot, uniform
    if (i == j) notpd = !(p > tol) || !__builtin_isfinite(p);
    const double r = rsqrt_f64(p > 0.0 ? p : 0.0);
    if (i == 0) rinv[j] = r;
    const double lij = (i >= j) ? a[j] * r : 0.0;
    a[j] = lij;
    Ls[i][j] = lij;
    Lc[j][i] = lij;
    // The block is one wavefront, whose LDS operations complete in issue order, so
    // wavefront-scope ordering makes the column visible to every lane without waiting
    // for the writes to finish before the reads are issued.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // a[i][l] -= L[i][j] L[l][j] for l > j.  Unguarded: lanes i < j have lij = 0, and the
    // entries l > i it writes lie above the diagonal, which are never read as pivots or
    // column entries (a[j] of lane i < j is replaced by lij = 0) nor stored.
#pragma unroll
    for (int l = j + 1; l < NB; ++l) a[l] = fma(-lij, Lc[j][l], a[l]);
  }
  if (notpd) atomicOr(flag, FLAG_NOTPD);
#pragma unroll
  for (int c = 0; c < NB; ++c)
    if (c <= i) A[(k0 + i) * lda + k0 + c] = a[c];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // Ls holds L (lower; entries above the diagonal are zero); rinv[r] = 1 / L[r][r]
  // X = L^{-1}, lane i holds column i: x[r] = (delta_ri - sum_{q<r} L[r][q] x[q]) / L[r][r]
  double x[NB];
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    double acc[4] = {(r == i) ? 1.0 : 0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < r; ++q) acc[q & 3] = fma(-Ls[r][q], x[q], acc[q & 3]);
    x[r] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * rinv[r];
  }
  double* __restrict__ out = Dinv + k * NB * NB;
#pragma unroll
  for (int r = 0; r < NB; ++r) out[r * NB + i] = (r >= i) ? x[r] : 0.0;
}

// Rows below block k:  A[i][k-block] <- A[i][k-block] * Dinv_k^T.  One 64-row tile
// per workgroup.
__global__ __launch_bounds__(kThreads) void panel_solve(double* __restrict__ A, int64_t lda, int64_t k,
                                                        const double* __restrict__ Dinv);

__device__ __forceinline__ void tri_tile(int64_t t, int64_t& ti, int64_t& tj) {
  // lower-triangle enumeration: (0,0), (1,0), (1,1), (2,0), ...
  int64_t i = static_cast<int64_t>((sqrt(8.0 * static_cast<double>(t) + 1.0) - 1.0) * 0.5);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// C[64x64 tile] -= A_op * B_op (STORE: C = A_op * B_op) with K = 64.
//  A_op[m][q] = A[(am0 + m) * lda + ak0 + q]
//  B_op[q][n] = BNN ? B[(bk0 + q) * ldb + bn0 + n] : B[(bn0 + n) * ldb + bk0 + q]
// Both operands are staged in LDS before any output is written, so C may alias them.
// Threads own 4 x 4 outputs (rows ty + 16a, cols tx + 16b).
template <bool BNN, bool STORE = false>
__device__ __forceinline__ void tile_update(double* __restrict__ C, int64_t ldc, int64_t cm0,
                                            int64_t cn0, const double* __restrict__ A, int64_t lda,
                                            int64_t am0, int64_t ak0, const double* __restrict__ B,
                                            int64_t ldb, int64_t bk0, int64_t bn0) {
  __shared__ double as[NB][NB + 1];   // [q][m]
  __shared__ double bs[NB][NB + 1];   // [q][n]
  const int tid = threadIdx.x;
  for (int e = tid; e < NB * NB; e += kThreads) {
    const int r = e / NB, c = e % NB;
    as[c][r] = A[(am0 + r) * lda + ak0 + c];              // A row r, k = c
    if (BNN) bs[r][c] = B[(bk0 + r) * ldb + bn0 + c];     // k = r, n = c
    else bs[c][r] = B[(bn0 + r) * ldb + bk0 + c];         // n = r, k = c
  }
  __syncthreads();
  const int tx = tid & 15, ty = tid >> 4;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int q = 0; q < NB; ++q) {
    double av[4], bv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) av[a] = as[q][ty + 16 * a];
#pragma unroll
    for (int b = 0; b < 4; ++b) bv[b] = bs[q][tx + 16 * b];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      double* c = C + (cm0 + ty + 16 * a) * ldc + cn0 + tx + 16 * b;
      if (STORE)
        *c = acc[a][b];
      else
        *c -= acc[a][b];
    }
}

__global__ __launch_bounds__(kThreads) void panel_solve(double* __restrict__ A, int64_t lda, int64_t k,
                                                        const double* __restrict__ Dinv) {
  const int64_t k0 = k * NB;
  const int64_t r0 = k0 + NB + static_cast<int64_t>(blockIdx.x) * NB;
  // out[i][c] = sum_q A[r0+i][k0+q] Dinv_k[c][q]
  tile_update<false, true>(A, lda, r0, k0, A, lda, r0, k0, Dinv + k * NB * NB, NB, 0, 0);
}

// Cholesky trailing update after block column k: lower tiles (ti >= tj) of the
// trailing matrix from block `first` on, A[i][j] -= L[i][k-block] L[j][k-block]^T.
__global__ __launch_bounds__(kThreads) void chol_trailing(double* __restrict__ A, int64_t lda, int64_t k,
                                                          int64_t first) {
  int64_t ti, tj;
  tri_tile(blockIdx.x, ti, tj);
  const int64_t base = first * NB;
  const int64_t i0 = base + ti * NB, j0 = base + tj * NB, k0 = k * NB;
  tile_update<false>(A, lda, i0, j0, A, lda, i0, k0, A, lda, k0, j0);
}

// The same update restricted to block column k + 1 (the next diagonal block's column).
__global__ __launch_bounds__(kThreads) void chol_trailing_col(double* __restrict__ A, int64_t lda,
                                                              int64_t k) {
  const int64_t j0 = (k + 1) * NB;
  const int64_t i0 = j0 + static_cast<int64_t>(blockIdx.x) * NB, k0 = k * NB;
  tile_update<false>(A, lda, i0, j0, A, lda, i0, k0, A, lda, k0, j0);
}

// Inverse step i, part 1: X[i][j-block] = Dinv_i * S[i][j-block] for j <= i, in place.
__global__ __launch_bounds__(kThreads) void inv_rowscale(double* __restrict__ X, int64_t ldx, int64_t i,
                                                         const double* __restrict__ Dinv) {
  const int64_t r0 = i * NB, c0 = static_cast<int64_t>(blockIdx.x) * NB;
  tile_update<true, true>(X, ldx, r0, c0, Dinv + i * NB * NB, NB, 0, 0, X, ldx, r0, c0);
}

// Inverse step i, part 2: S[r][j] -= L[r][i] X[i][j] for block rows r > i, j <= i.
__global__ __launch_bounds__(kThreads) void inv_update(double* __restrict__ X, int64_t ldx,
                                                       const double* __restrict__ L, int64_t ldl,
                                                       int64_t i) {
  const int64_t ncol = i + 1;
  const int64_t rb = i + 1 + blockIdx.x / ncol;
  const int64_t jb = blockIdx.x % ncol;
  tile_update<true>(X, ldx, rb * NB, jb * NB, L, ldl, rb * NB, i * NB, X, ldx, i * NB, jb * NB);
}

__global__ __launch_bounds__(kThreads) void fill_identity(double* __restrict__ X, int64_t ld) {
  const int64_t total = ld * ld;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x)
    X[e] = (e / ld == e % ld) ? 1.0 : 0.0;
}

// Rt[a][b] = R[b][a] = Linv[d-1-b][d-1-a] (zero above the diagonal), fp32.
__global__ __launch_bounds__(kThreads) void extract_rt(const double* __restrict__ X, int64_t ldx,
                                                       int64_t d, float* __restrict__ Rt, int64_t ldr) {
  const int64_t total = d * d;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t a = e / d, b = e % d;
    Rt[a * ldr + b] = (b <= a) ? static_cast<float>(X[(d - 1 - b) * ldx + (d - 1 - a)]) : 0.0f;
  }
}

inline unsigned grid_for(int64_t n) {
  int64_t b = ceil_div(n, kThreads * 4);
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return static_cast<unsigned>(b);
}

}  // namespace

size_t rfactor_ws_bytes(int64_t d) {
  const int64_t dp = round_up(d < 1 ? 1 : d, NB);
  const int64_t nblk = dp / NB;
  size_t b = 0;
  b += align256(static_cast<size_t>(dp) * dp * sizeof(double));   // A -> L
  b += align256(static_cast<size_t>(dp) * dp * sizeof(double));   // S -> X = L^{-1}
  b += align256(static_cast<size_t>(nblk) * NB * NB * sizeof(double));
  b += align256(static_cast<size_t>(dp) * sizeof(double));
  return b;
}

namespace {

// Streams and events for the look-ahead schedule, created once per host thread and
// device (default priority; kept until the process ends).  When they cannot be created
// every launch goes to the caller's stream.
struct Lookahead {
  int device = -1;
  bool ok = false;
  hipStream_t trail = nullptr, inv = nullptr;
  hipEvent_t ev_panel = nullptr, ev_trail = nullptr, ev_join1 = nullptr, ev_join2 = nullptr;
};

Lookahead* lookahead() {
  thread_local std::vector<Lookahead> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  for (Lookahead& l : cache)
    if (l.device == dev) return l.ok ? &l : nullptr;
  Lookahead l;
  l.device = dev;
  l.ok = hipStreamCreateWithFlags(&l.trail, hipStreamNonBlocking) == hipSuccess &&
         hipStreamCreateWithFlags(&l.inv, hipStreamNonBlocking) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_panel, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_trail, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_join1, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_join2, hipEventDisableTiming) == hipSuccess;
  cache.push_back(l);
  return cache.back().ok ? &cache.back() : nullptr;
}

// The reversed-order Cholesky in place, A (lower) = L with L L^T = J Hp J, plus the
// inverses of the diagonal blocks in Dinv and, when X is given, X = L^{-1}.
//
// Look-ahead schedule.  The caller's stream runs the critical chain: per block column
// k the diagonal block, the panel below it, and the trailing update of block column
// k + 1 only (all the next diagonal block needs).  A second stream applies block column
// k to the rest of the trailing matrix (columns >= k + 2) while the chain moves on; a
// third runs inverse step k (X row block k and its update of the rows below) as soon as
// the panel of k is done.  The update of column k + 1 waits for the previous step's
// rest update, so every tile still receives its updates in order of k, and the results
// are those of the one-stream order.
int factor_reversed(const float* H, int64_t d, const int32_t* perm, double* A, int64_t dp,
                    double* Dinv, double* diag0, double* X, uint32_t* flag, hipStream_t s) {
  const int64_t nblk = dp / NB;
  Lookahead* la = lookahead();
  hipStream_t s_trail = la ? la->trail : s, s_inv = la ? la->inv : s;
  auto fork = [&](hipStream_t to, hipEvent_t ev) -> int {
    if (!la) return QZ_OK;
    QZ_HIP(hipStreamWaitEvent(to, ev, 0));
    return QZ_OK;
  };
  auto mark = [&](hipEvent_t ev, hipStream_t on) -> int {
    if (!la) return QZ_OK;
    QZ_HIP(hipEventRecord(ev, on));
    return QZ_OK;
  };
  init_reversed<<<grid_for(dp * dp), kThreads, 0, s>>>(H, d, perm, A, dp, diag0, flag);
  QZ_TRY(check_launch("rfactor.init"));
  if (X) {
    fill_identity<<<grid_for(dp * dp), kThreads, 0, s>>>(X, dp);
    QZ_TRY(check_launch("rfactor.fill"));
  }
  for (int64_t k = 0; k < nblk; ++k) {
    const int64_t below = nblk - k - 1;
    diag_block<<<1, NB, 0, s>>>(A, dp, k, diag0, Dinv, flag);
    QZ_TRY(check_launch("rfactor.diag"));
    if (below > 0) {
      panel_solve<<<static_cast<unsigned>(below), kThreads, 0, s>>>(A, dp, k, Dinv);
      QZ_TRY(check_launch("rfactor.panel"));
    }
    QZ_TRY(mark(la ? la->ev_panel : nullptr, s));
    QZ_TRY(fork(s_trail, la ? la->ev_panel : nullptr));
    if (X) QZ_TRY(fork(s_inv, la ? la->ev_panel : nullptr));
    if (below > 0) {
      if (k > 0) QZ_TRY(fork(s, la ? la->ev_trail : nullptr));   // rest update of k - 1 done
      chol_trailing_col<<<static_cast<unsigned>(below), kThreads, 0, s>>>(A, dp, k);
      QZ_TRY(check_launch("rfactor.trailing_col"));
    }
    if (below > 1) {
      chol_trailing<<<static_cast<unsigned>((below - 1) * below / 2), kThreads, 0, s_trail>>>(
          A, dp, k, k + 2);
      QZ_TRY(check_launch("rfactor.trailing"));
    }
    QZ_TRY(mark(la ? la->ev_trail : nullptr, s_trail));
    if (X) {
      inv_rowscale<<<static_cast<unsigned>(k + 1), kThreads, 0, s_inv>>>(X, dp, k, Dinv);
      QZ_TRY(check_launch("rfactor.rowscale"));
      if (below > 0) {
        inv_update<<<static_cast<unsigned>(below * (k + 1)), kThreads, 0, s_inv>>>(X, dp, A, dp, k);
        QZ_TRY(check_launch("rfactor.invupdate"));
      }
    }
  }
  // join: the caller's stream continues after both side streams
  QZ_TRY(mark(la ? la->ev_join1 : nullptr, s_trail));
  QZ_TRY(fork(s, la ? la->ev_join1 : nullptr));
  if (X) {
    QZ_TRY(mark(la ? la->ev_join2 : nullptr, s_inv));
    QZ_TRY(fork(s, la ? la->ev_join2 : nullptr));
  }
  return QZ_OK;
}

// D[j] = L[d-1-j][d-1-j]^2: the LDL pivot of the column quantized j-th.
__global__ void pivots_from_factor(const double* __restrict__ A, int64_t lda, int64_t d,
                                   double* __restrict__ D) {
  for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < d;
       j += (int64_t)gridDim.x * blockDim.x) {
    const double l = A[(d - 1 - j) * lda + (d - 1 - j)];
    D[j] = l * l;
  }
}

}  // namespace

int rfactor(const float* H, int64_t d, const int32_t* perm, float* Rt, int64_t ldr, void* ws,
            uint32_t* flag, hipStream_t s) {
  const int64_t dp = round_up(d, NB);
  const int64_t nblk = dp / NB;
  Carver cv(ws);
  double* A = cv.take<double>(static_cast<size_t>(dp) * dp);
  double* X = cv.take<double>(static_cast<size_t>(dp) * dp);
  double* Dinv = cv.take<double>(static_cast<size_t>(nblk) * NB * NB);
  double* diag0 = cv.take<double>(static_cast<size_t>(dp));
  QZ_TRY(factor_reversed(H, d, perm, A, dp, Dinv, diag0, X, flag, s));
  extract_rt<<<grid_for(d * d), kThreads, 0, s>>>(X, dp, d, Rt, ldr);
  return check_launch("rfactor.extract");
}

int order_pivots(const float* H, int64_t d, const int32_t* perm, double* D, void* ws,
                 uint32_t* flag, hipStream_t s) {
  const int64_t dp = round_up(d, NB);
  const int64_t nblk = dp / NB;
  Carver cv(ws);
  double* A = cv.take<double>(static_cast<size_t>(dp) * dp);
  cv.take<double>(static_cast<size_t>(dp) * dp);   // (the inverse's buffer, unused here)
  double* Dinv = cv.take<double>(static_cast<size_t>(nblk) * NB * NB);
  double* diag0 = cv.take<double>(static_cast<size_t>(dp));
  QZ_TRY(factor_reversed(H, d, perm, A, dp, Dinv, diag0, nullptr, flag, s));
  pivots_from_factor<<<grid_for(d), kThreads, 0, s>>>(A, dp, d, D);
  return check_launch("order_pivots");
}

}  // namespace qz
