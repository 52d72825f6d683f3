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

// A[i][j] = Hp[d-1-i][d-1-j] (Hp = H[perm][:, perm]) for i, j < d, identity padding, over
// the block columns jb0 <= j / 64 < jb1 (all rows).  Only the tiles on or below the diagonal
// are written (the factorisation reads no others); every entry of H in those columns is
// checked.
__global__ __launch_bounds__(kThreads) void init_reversed(const float* __restrict__ H, int64_t d,
                                                          const int32_t* __restrict__ perm,
                                                          double* __restrict__ A, int64_t lda,
                                                          int64_t jb0, int64_t jb1,
                                                          double* __restrict__ diag0,
                                                          uint32_t* __restrict__ flag) {
  const int64_t w = (jb1 - jb0) * NB;
  const int64_t total = lda * w;
  bool bad = false;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / w, j = jb0 * NB + e % w;
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
    if (j / NB <= i / NB) A[i * lda + j] = v;
    if (i == j) diag0[i] = v;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, FLAG_NONFINITE);
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), l);
  return __hiloint2double(hi, lo);
}

// orders this wavefront's LDS accesses (its LDS operations complete in order)
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 1 / sqrt(p) for p > 0: the hardware estimate refined by two Newton steps
// y <- y (3 - p y^2) / 2 (each step squares the relative error).
__device__ __forceinline__ double rsqrt_f64(double p) {
  double y = __builtin_amdgcn_rsq(p);
  y = y * (1.5 - 0.5 * p * y * y);
  y = y * (1.5 - 0.5 * p * y * y);
  return y;
}

// Factor diagonal block k in place (lower) and write its inverse to Dinv[k]: four
// wavefronts, the block held in LDS and factored right-looking over four 16-column panels:
//   (1) wavefront 0 factors the panel's rows c0 .. 63, one lane per row holding the row's
//       16 panel entries in registers: per pivot j the pivot comes from lane j by readlane,
//       each lane scales its own entry (L[i][j]) and writes it to LDS, and updates its later
//       entries with the column values L[c][j] (the next column's by readlane, the others
//       read back from LDS at uniform addresses).  The rows below the 16 x 16 diagonal
//       sub-block are solved by the same instructions;
//   (2) all four wavefronts update the trailing lower triangle, A[i][j] -= sum over the
//       panel of L[i][m] L[j][m], in 16 x 16 blocks on the matrix cores; one barrier
//       before (2), one after.
// The inverse X = L^{-1}, in 16 x 16 blocks, formed by the other wavefronts while wavefront
// 0 runs the next panel's chain: the diagonal block of panel p by wavefront 1 during chain
// p + 1 (one lane per column, forward substitution; the last panel's by wavefront 0 inside
// its own chain), row block R below the diagonal, X_Rq = -X_RR sum_{q <= m < R} L_Rm X_mq,
// by wavefronts 2 and 3 on the matrix cores during chain R + 2 (row blocks 2 and 3 after
// the loop).  Entries above the diagonal are never read as pivots or L entries and are
// not stored.
typedef double v4f64 __attribute__((ext_vector_type(4)));

constexpr int PB = 16;                  // panel width
constexpr int kDiagThreads = 256;
constexpr int LS = NB + 1;              // LDS row stride of the block (doubles)

// LDS of the diagonal factorisation, in doubles: the block (then L), X = L^{-1}, the pivot
// tolerances and the reciprocal pivots.
constexpr int kTolOff = 2 * NB * LS;
constexpr int kRinvOff = kTolOff + NB;   // 1 / L[r][r]
constexpr int kDiagLds = kRinvOff + NB;

// Diagonal block R of X = L^{-1} (16 x 16, one wavefront, lane c < 16 forming column c by
// forward substitution: x[r] = (delta_rc - sum_{m<r} L[r][m] x[m]) / L[r][r]).  The same
// operations in the same order as the form inside the pivot chain.
__device__ __forceinline__ void x_diag(const double* S, double* Xf, const double* rinv, int R,
                                       int lane) {
  if (lane < PB) {
    const int b0 = PB * R;
    double x[PB];
#pragma unroll
    for (int r = 0; r < PB; ++r) {
      double xa = (r == lane) ? 1.0 : 0.0;
#pragma unroll
      for (int m = 0; m < r; ++m) xa = fma(-S[(b0 + r) * LS + b0 + m], x[m], xa);
      x[r] = (r >= lane) ? xa * rinv[b0 + r] : 0.0;
    }
#pragma unroll
    for (int r = 0; r < PB; ++r) Xf[(b0 + r) * LS + b0 + lane] = x[r];
  }
}

// Row block R, column block q < R of X = L^{-1} (16 x 16 blocks, one wavefront):
// X_Rq = -X_RR sum_{q <= m < R} L_Rm X_mq, with L in S and the blocks X_mq (m < R) and
// X_RR already in Xf.  Both products run on v_mfma_f64_16x16x4; the second one's right
// operand fragments are the first one's result registers (element i of lane l is row
// l / 16 + 4 i, column l % 16, which is what step k = 4 i of the next product reads).
__device__ __forceinline__ void x_offdiag(const double* S, double* Xf, int R, int q, int lane) {
  const int lr = lane >> 4, lc = lane & 15;
  v4f64 tb = v4f64{0.0, 0.0, 0.0, 0.0};
  for (int m = q; m < R; ++m) {
#pragma unroll
    for (int k0 = 0; k0 < PB; k0 += 4) {
      const double a = S[(PB * R + lc) * LS + PB * m + k0 + lr];
      const double b = Xf[(PB * m + k0 + lr) * LS + PB * q + lc];
      tb = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, tb, 0, 0, 0);
    }
  }
  v4f64 xr = v4f64{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double a = Xf[(PB * R + lc) * LS + PB * R + 4 * i + lr];
    xr = __builtin_amdgcn_mfma_f64_16x16x4f64(a, tb[i], xr, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) Xf[(PB * R + lr + 4 * i) * LS + PB * q + lc] = -xr[i];
}

// Diagonal block k of A into S (the LDS block of the factorisation, lower part, zero above the
// diagonal) and the pivot tolerances into tolv.  All 16 loads of a thread are in flight at
// once (every address lies inside A).
__device__ __forceinline__ void diag_load(const double* __restrict__ A, int64_t lda, int64_t k,
                                          const double* __restrict__ diag0, double* smem) {
  double* S = smem;
  double* tolv = smem + kTolOff;
  const int tid = threadIdx.x;
  const int64_t k0 = k * NB;
  constexpr int PER = NB * NB / kDiagThreads;
  double v[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int e = tid + t * kDiagThreads;
    v[t] = A[(k0 + e / NB) * lda + k0 + e % NB];
  }
  if (tid < NB) tolv[tid] = 1e-12 * diag0[k0 + tid];
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int e = tid + t * kDiagThreads;
    const int i = e / NB, c = e % NB;
    S[i * LS + c] = (c <= i) ? v[t] : 0.0;
  }
}

// Factor the block held in S (and tolv) as above, write L to diagonal block k of A and
// L^{-1} to Dinv[k].  The caller has filled S and tolv and passed a barrier.
__device__ __forceinline__ void diag_factor_lds(double* __restrict__ A, int64_t lda, int64_t k,
                                                double* __restrict__ Dinv,
                                                uint32_t* __restrict__ flag, double* smem) {
  double* S = smem;                           // the block, then L (lower)
  double* Xf = S + NB * LS;                   // X = L^{-1}
  const double* tolv = smem + kTolOff;        // 1e-12 of the original diagonal
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t k0 = k * NB;

  bool notpd = false;
  double* rinv = smem + kRinvOff;
#pragma unroll 1
  for (int c0 = 0; c0 < NB; c0 += PB) {
    const int pb = c0 / PB;
    const bool last = c0 + PB == NB;
    if (wave == 0) {
      // (1) the panel's rows c0 .. 63, one lane per row, 16 entries in registers; in the last
      // panel lane c < 16 also forms column c of the inverse of the 16 x 16 diagonal
      // sub-block, row j right after pivot j (row j of L is final then)
      const bool act = lane < NB - c0;
      const int i = c0 + (act ? lane : 0);
      double v[PB], x[PB];
#pragma unroll
      for (int m = 0; m < PB; ++m) v[m] = act ? S[i * LS + c0 + m] : 0.0;
      const double tol = act ? tolv[i] : 0.0;
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const double p = readlane_f64(v[j], j);               // pivot, uniform
        notpd = notpd || (lane == j && (!(p > tol) || !__builtin_isfinite(p)));
        const double rj = rsqrt_f64(p > 0.0 ? p : 0.0);
        const double t = (act && lane >= j) ? v[j] * rj : 0.0;   // L[i][c0 + j]
        v[j] = t;
        if (act) S[i * LS + c0 + j] = t;                         // column j of L, in place
        if (lane == 0) rinv[c0 + j] = rj;
        wave_sync_lds();
        // the next pivot's column first; the other column values come back from LDS as
        // uniform reads
        if (j + 1 < PB) v[j + 1] = fma(-t, readlane_f64(t, j + 1), v[j + 1]);
#pragma unroll
        for (int c = j + 2; c < PB; ++c) v[c] = fma(-t, S[(c0 + c) * LS + c0 + j], v[c]);
        if (last) {
          double xa = (lane == j) ? 1.0 : 0.0;
#pragma unroll
          for (int m = 0; m < j; ++m) xa = fma(-S[(c0 + j) * LS + c0 + m], x[m], xa);
          x[j] = (j >= lane) ? xa * rj : 0.0;
        }
      }
      if (last && lane < PB) {
#pragma unroll
        for (int r = 0; r < PB; ++r) Xf[(c0 + r) * LS + c0 + lane] = x[r];
      }
    } else if (wave == 1) {
      // meanwhile: the previous panel's diagonal block of the inverse
      if (pb >= 1) x_diag(S, Xf, rinv, pb - 1, lane);
    } else if (wave - 2 < pb - 2) {
      // and row block pb - 2 of the inverse, column block wave - 2
      x_offdiag(S, Xf, pb - 2, wave - 2, lane);
    }
    __syncthreads();
    // (2) trailing lower triangle, rows and columns c0 + 16 .. 63, in 16 x 16 blocks on the
    // matrix cores (K = 16: four v_mfma_f64_16x16x4)
    const int nbt = (NB - c0 - PB) / 16;
    const int lr = lane >> 4, lc = lane & 15;
    for (int t = wave; t < nbt * (nbt + 1) / 2; t += kDiagThreads / 64) {
      int bi = 0;
      while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
      const int bj = t - bi * (bi + 1) / 2;
      const int rb = c0 + PB + 16 * bi, cb = c0 + PB + 16 * bj;
      v4f64 acc = v4f64{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int k0 = 0; k0 < PB; k0 += 4) {
        const double a = S[(rb + lc) * LS + c0 + k0 + lr];
        const double bb = S[(cb + lc) * LS + c0 + k0 + lr];
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bb, acc, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) S[(rb + lr + 4 * q) * LS + cb + lc] -= acc[q];
    }
    __syncthreads();
  }
  // the last two row blocks of the inverse: row block 2 (its diagonal block came from the
  // last panel's phase), then row block 3 (its diagonal block from the last chain)
  if (wave >= 2) x_offdiag(S, Xf, NB / PB - 2, wave - 2, lane);
  __syncthreads();
  // the last row block of the inverse
  if (wave < NB / PB - 1) x_offdiag(S, Xf, NB / PB - 1, wave, lane);
  if (__any(notpd) && tid == 0) atomicOr(flag, FLAG_NOTPD);

#pragma unroll
  for (int t = 0; t < NB * NB / kDiagThreads; ++t) {
    const int e = tid + t * kDiagThreads;
    const int i = e / NB, c = e % NB;
    if (c <= i) A[(k0 + i) * lda + k0 + c] = S[i * LS + c];
  }
  __syncthreads();
  double* __restrict__ out = Dinv + k * NB * NB;
#pragma unroll
  for (int t = 0; t < NB * NB / kDiagThreads; ++t) {
    const int e = tid + t * kDiagThreads;
    const int rr = e / NB, cc = e % NB;
    out[e] = (rr >= cc) ? Xf[rr * LS + cc] : 0.0;
  }
}

__device__ __forceinline__ void tri_tile(int64_t t, int64_t& ti, int64_t& tj) {
  // lower-triangle enumeration: (0,0), (1,0), (1,1), (2,0), ...
  int64_t i = static_cast<int64_t>((sqrt(8.0 * static_cast<double>(t) + 1.0) - 1.0) * 0.5);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// C[64x64 tile] -= A_op * B_op (STORE: C = A_op * B_op) with K = 64, on the fp64 matrix
// cores.
//  A_op[m][q] = A[(am0 + m) * lda + ak0 + q]
//  B_op[q][n] = BNN ? B[(bk0 + q) * ldb + bn0 + n] : B[(bn0 + n) * ldb + bk0 + q]
// Both operands are staged in LDS before any output is written, so C may alias them.
// Every thread issues all of its operand loads (and, when updating, its 16 loads of C)
// before waiting for any of them.  Wavefront w computes the 32 x 32 quadrant at rows
// 32 (w / 2), columns 32 (w % 2) as 2 x 2 blocks of v_mfma_f64_16x16x4 (16 x 4 times
// 4 x 16 per instruction, 16 instructions along K).  Fragment layout of that instruction
// (lane l): A[l % 16][l / 16], B[l / 16][l % 16], and result element i at D[l / 16 + 4 i]
// [l % 16].  The products are summed from zero and subtracted from C once at the end.
template <bool BNN, bool STORE = false, bool TO_S = false>
__device__ __forceinline__ void tile_update_lds(double* __restrict__ C, int64_t ldc, int64_t cm0,
                                                int64_t cn0, const double* __restrict__ A,
                                                int64_t lda, int64_t am0, int64_t ak0,
                                                const double* __restrict__ B, int64_t ldb,
                                                int64_t bk0, int64_t bn0, double* smem) {
  typedef double Row[NB + 1];
  Row* as = reinterpret_cast<Row*>(smem);                  // [q][m]
  Row* bs = reinterpret_cast<Row*>(smem + NB * (NB + 1));  // [q][n]
  constexpr int PER = NB * NB / kThreads;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane >> 4, lc = lane & 15;
  const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32;
  double va[PER], vb[PER], cv[2][2][4];
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int e = tid + t * kThreads;
    const int r = e / NB, c = e % NB;
    va[t] = A[(am0 + r) * lda + ak0 + c];                                       // A row r, k = c
    vb[t] = BNN ? B[(bk0 + r) * ldb + bn0 + c] : B[(bn0 + r) * ldb + bk0 + c];   // (k, n) = (r, c) or (c, r)
  }
  if (!STORE) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          cv[a][b][i] = C[(cm0 + r0 + 16 * a + lr + 4 * i) * ldc + cn0 + c0 + 16 * b + lc];
  }
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int e = tid + t * kThreads;
    const int r = e / NB, c = e % NB;
    as[c][r] = va[t];
    if (BNN) bs[r][c] = vb[t];
    else bs[c][r] = vb[t];
  }
  __syncthreads();
  v4f64 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = v4f64{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int q = 0; q < NB; q += 4) {
    const double a0 = as[q + lr][r0 + lc], a1 = as[q + lr][r0 + 16 + lc];
    const double b0 = bs[q + lr][c0 + lc], b1 = bs[q + lr][c0 + 16 + lc];
    acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
  }
  if (TO_S) {
    // the updated tile goes to the LDS block of the diagonal factorisation instead (lower
    // part, zero above the diagonal), over the staging area once every wavefront is done
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = r0 + 16 * a + lr + 4 * i, n = c0 + 16 * b + lc;
          smem[m * LS + n] = (n <= m) ? cv[a][b][i] - acc[a][b][i] : 0.0;
        }
    return;
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        double* c = C + (cm0 + r0 + 16 * a + lr + 4 * i) * ldc + cn0 + c0 + 16 * b + lc;
        *c = STORE ? acc[a][b][i] : cv[a][b][i] - acc[a][b][i];
      }
}

template <bool BNN, bool STORE = false>
__device__ __forceinline__ void tile_update(double* __restrict__ C, int64_t ldc, int64_t cm0,
                                            int64_t cn0, const double* __restrict__ A, int64_t lda,
                                            int64_t am0, int64_t ak0, const double* __restrict__ B,
                                            int64_t ldb, int64_t bk0, int64_t bn0) {
  __shared__ double smem[2 * NB * (NB + 1)];
  tile_update_lds<BNN, STORE>(C, ldc, cm0, cn0, A, lda, am0, ak0, B, ldb, bk0, bn0, smem);
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

// The same update for one block column c only: tiles (c + blockIdx.x, c).
__global__ __launch_bounds__(kThreads) void chol_trailing_col(double* __restrict__ A, int64_t lda,
                                                              int64_t k, int64_t c) {
  const int64_t i0 = (c + static_cast<int64_t>(blockIdx.x)) * NB, j0 = c * NB, k0 = k * NB;
  tile_update<false>(A, lda, i0, j0, A, lda, i0, k0, A, lda, k0, j0);
}

// Rows below block k:  A[i][k-block] <- A[i][k-block] * Dinv_k^T, in place.  16 rows per
// workgroup, one 16 x 16 output block per wavefront (16 v_mfma_f64_16x16x4 along K), the
// fragments read straight from global memory (A_op[m][q] from row r0 + m, B_op[q][n] =
// Dinv_k[n][q]), with the fragment layout and K order of tile_update_lds, so the results are
// those of the 64-row tile product.  Every wavefront reads all 64 columns of the rows before
// any wavefront writes its 16.
__global__ __launch_bounds__(kThreads) void panel_solve(double* __restrict__ A, int64_t lda, int64_t k,
                                                        const double* __restrict__ Dinv) {
  const int64_t k0 = k * NB;
  const int64_t r0 = k0 + NB + static_cast<int64_t>(blockIdx.x) * 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane >> 4, lc = lane & 15;
  const double* __restrict__ Dk = Dinv + k * NB * NB;
  double a[NB / 4], b[NB / 4];
#pragma unroll
  for (int s = 0; s < NB / 4; ++s) {
    a[s] = A[(r0 + lc) * lda + k0 + 4 * s + lr];
    b[s] = Dk[(16 * w + lc) * NB + 4 * s + lr];
  }
  v4f64 acc = v4f64{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < NB / 4; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], b[s], acc, 0, 0, 0);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) A[(r0 + lr + 4 * i) * lda + k0 + 16 * w + lc] = acc[i];
}

// The update of block column k + 1 by panel k, A(i,k+1) -= L(i,k) L(k+1,k)^T for the block
// rows i > k, and then, in workgroup 0 (whose tile is the next diagonal block), the
// factorisation and inverse of diagonal block k + 1: one launch on the critical chain.  With
// k = -1 (one workgroup) it only factors diagonal block 0, read from A.
constexpr int kStepLds = (kDiagLds > 2 * NB * (NB + 1)) ? kDiagLds : 2 * NB * (NB + 1);
// Extra dynamic LDS for this launch: with it, no workgroup of the 64 x 64 tile kernels
// (66.5 KB each) fits on the compute unit beside the diagonal factorisation, which
// therefore runs alone on its unit.
constexpr size_t kStepPadBytes = 30720;

__global__ __launch_bounds__(kThreads) void col_diag(double* __restrict__ A, int64_t lda, int64_t k,
                                                     const double* __restrict__ diag0,
                                                     double* __restrict__ Dinv,
                                                     uint32_t* __restrict__ flag) {
  __shared__ double smem[kStepLds];
  const int64_t j0 = (k + 1) * NB;
  const int64_t i0 = j0 + static_cast<int64_t>(blockIdx.x) * NB, k0 = k * NB;
  if (blockIdx.x == 0) {
    if (k < 0) {
      diag_load(A, lda, 0, diag0, smem);
    } else {
      // the diagonal tile's update lands in LDS, where its factorisation reads it
      if (threadIdx.x < NB) smem[kTolOff + threadIdx.x] = 1e-12 * diag0[j0 + threadIdx.x];
      tile_update_lds<false, false, true>(A, lda, i0, j0, A, lda, i0, k0, A, lda, k0, j0, smem);
    }
    __syncthreads();
    diag_factor_lds(A, lda, k + 1, Dinv, flag, smem);
  } else {
    tile_update_lds<false>(A, lda, i0, j0, A, lda, i0, k0, A, lda, k0, j0, smem);
  }
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

// X = I on the tiles on or below the diagonal (the only ones the inverse reads).
__global__ __launch_bounds__(kThreads) void fill_identity(double* __restrict__ X, int64_t ld) {
  const int64_t total = ld * ld;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / ld, j = e % ld;
    if (j / NB <= i / NB) X[e] = (i == j) ? 1.0 : 0.0;
  }
}

// Rt[a][b] = R[b][a] = Linv[d-1-b][d-1-a] (zero above the diagonal), fp32.  One 64 x 64
// tile of Rt per workgroup (grid: column tiles x row tiles), transposed through LDS so that
// both the reads of X and the writes of Rt are coalesced; tiles above the diagonal are only
// zero-filled.
__global__ __launch_bounds__(kThreads) void extract_rt(const double* __restrict__ X, int64_t ldx,
                                                       int64_t d, float* __restrict__ Rt, int64_t ldr) {
  __shared__ float t[NB][NB + 1];
  const int64_t a0 = static_cast<int64_t>(blockIdx.y) * NB, b0 = static_cast<int64_t>(blockIdx.x) * NB;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  if (b0 <= a0) {
#pragma unroll
    for (int s = 0; s < NB / 4; ++s) {
      const int by = ty + 4 * s;
      const int64_t a = a0 + tx, b = b0 + by;
      // X row d-1-b, column d-1-a: consecutive lanes read consecutive (descending) columns
      t[by][tx] = (a < d && b < d && b <= a) ? static_cast<float>(X[(d - 1 - b) * ldx + (d - 1 - a)]) : 0.0f;
    }
    __syncthreads();
  }
#pragma unroll
  for (int s = 0; s < NB / 4; ++s) {
    const int ay = ty + 4 * s;
    const int64_t a = a0 + ay, b = b0 + tx;
    if (a < d && b < d) Rt[a * ldr + b] = (b0 <= a0) ? t[tx][ay] : 0.0f;
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
  b += align256(static_cast<size_t>(nblk) * NB * NB * sizeof(double));   // Dinv
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
  hipEvent_t ev_start = nullptr, ev_panel = nullptr, ev_trail = nullptr, ev_join1 = nullptr,
            ev_join2 = nullptr;
  hipStream_t side = nullptr;                        // work beside the factorisation
  hipEvent_t ev_fork = nullptr, ev_back = nullptr;
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
         hipStreamCreateWithFlags(&l.side, hipStreamNonBlocking) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_start, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_panel, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_trail, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_join1, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_join2, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_fork, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&l.ev_back, hipEventDisableTiming) == hipSuccess;
  cache.push_back(l);
  return cache.back().ok ? &cache.back() : nullptr;
}

}  // namespace

// A stream for work that may run beside the factorisation: `s` itself when the library's
// streams are unavailable; otherwise a stream of its own (not one the factorisation
// uses), made to wait for everything enqueued on `s` so far.  side_join makes `s` wait
// for what was enqueued there since.
int side_fork(hipStream_t s, hipStream_t* side) {
  Lookahead* la = lookahead();
  *side = s;
  if (!la) return QZ_OK;
  QZ_HIP(hipEventRecord(la->ev_fork, s));
  QZ_HIP(hipStreamWaitEvent(la->side, la->ev_fork, 0));
  *side = la->side;
  return QZ_OK;
}

int side_join(hipStream_t s, hipStream_t side) {
  if (side == s) return QZ_OK;
  Lookahead* la = lookahead();
  if (!la) return QZ_OK;
  QZ_HIP(hipEventRecord(la->ev_back, side));
  QZ_HIP(hipStreamWaitEvent(s, la->ev_back, 0));
  return QZ_OK;
}

namespace {

// The reversed-order Cholesky in place, A (lower) = L with L L^T = J Hp J, plus the
// inverses of the diagonal blocks in Dinv and, when X is given, X = L^{-1}.
//
// Look-ahead schedule.  The caller's stream runs the critical chain: per block column
// k the panel below diagonal block k, then one launch (col_diag) that updates block
// column k + 1 and factors diagonal block k + 1.  A second stream applies block column k
// to the rest of the trailing matrix (columns >= k + 2, column k + 2 first, the chain's next
// step waiting only for that column) while the chain moves on; a third
// runs inverse step k (X row block k and its update of the rows below) as soon as the
// panel of k is done.  The update of column k + 1 waits for the previous step's update of
// that column, which the rest-update stream runs after every earlier rest update, so every
// tile still receives its updates in order of k, and the results are those of the
// one-stream order.
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
  // The side streams start after all earlier work on s (which may still read A or X).  The
  // chain needs block columns 0 and 1 of A first; the init of the others runs on the rest
  // update's stream, ahead of the first rest update, and X = I on the inverse's stream.
  QZ_TRY(mark(la ? la->ev_start : nullptr, s));
  QZ_TRY(fork(s_trail, la ? la->ev_start : nullptr));
  if (X) {
    QZ_TRY(fork(s_inv, la ? la->ev_start : nullptr));
    fill_identity<<<grid_for(dp * dp), kThreads, 0, s_inv>>>(X, dp);
    QZ_TRY(check_launch("rfactor.fill"));
  }
  const int64_t near = nblk < 2 ? nblk : 2;
  init_reversed<<<grid_for(dp * near * NB), kThreads, 0, s>>>(H, d, perm, A, dp, 0, near, diag0,
                                                              flag);
  QZ_TRY(check_launch("rfactor.init"));
  if (nblk > near) {
    init_reversed<<<grid_for(dp * (nblk - near) * NB), kThreads, 0, s_trail>>>(
        H, d, perm, A, dp, near, nblk, diag0, flag);
    QZ_TRY(check_launch("rfactor.init2"));
  }
  col_diag<<<1, kThreads, kStepPadBytes, s>>>(A, dp, -1, diag0, Dinv, flag);
  QZ_TRY(check_launch("rfactor.diag"));
  for (int64_t k = 0; k < nblk; ++k) {
    const int64_t below = nblk - k - 1;
    if (below > 0) {
      panel_solve<<<static_cast<unsigned>(4 * below), kThreads, 0, s>>>(A, dp, k, Dinv);
      QZ_TRY(check_launch("rfactor.panel"));
    }
    QZ_TRY(mark(la ? la->ev_panel : nullptr, s));
    QZ_TRY(fork(s_trail, la ? la->ev_panel : nullptr));
    if (X) QZ_TRY(fork(s_inv, la ? la->ev_panel : nullptr));
    if (below > 0) {
      if (k > 0) QZ_TRY(fork(s, la ? la->ev_trail : nullptr));   // column k + 1 by panel k - 1
      col_diag<<<static_cast<unsigned>(below), kThreads, kStepPadBytes, s>>>(A, dp, k, diag0, Dinv,
                                                                           flag);
      QZ_TRY(check_launch("rfactor.coldiag"));
    }
    // Rest update by panel k: block column k + 2 first (the next step's col_diag waits for
    // it, and through the stream for the earlier rest updates), then the columns after it,
    // which have two chain steps to finish before the step that needs them.
    if (below > 1) {
      chol_trailing_col<<<static_cast<unsigned>(below - 1), kThreads, 0, s_trail>>>(A, dp, k,
                                                                                  k + 2);
      QZ_TRY(check_launch("rfactor.trailing_col"));
    }
    QZ_TRY(mark(la ? la->ev_trail : nullptr, s_trail));
    if (below > 2) {
      chol_trailing<<<static_cast<unsigned>((below - 2) * (below - 1) / 2), kThreads, 0,
                      s_trail>>>(A, dp, k, k + 3);
      QZ_TRY(check_launch("rfactor.trailing"));
    }
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

namespace {

int rfactor_enqueue(const float* H, int64_t d, const int32_t* perm, float* Rt, int64_t ldr,
                    void* ws, uint32_t* flag, hipStream_t s) {
  const int64_t dp = round_up(d, NB);
  const int64_t nblk = dp / NB;
  Carver cv(ws);
  double* A = cv.take<double>(static_cast<size_t>(dp) * dp);
  double* X = cv.take<double>(static_cast<size_t>(dp) * dp);
  double* Dinv = cv.take<double>(static_cast<size_t>(nblk) * NB * NB);
  double* diag0 = cv.take<double>(static_cast<size_t>(dp));
  QZ_TRY(factor_reversed(H, d, perm, A, dp, Dinv, diag0, X, flag, s));
  const unsigned nt = static_cast<unsigned>(ceil_div(d, NB));
  extract_rt<<<dim3(nt, nt), kThreads, 0, s>>>(X, dp, d, Rt, ldr);
  return check_launch("rfactor.extract");
}

// The R factor enqueues about 11 operations per 64-column step (launches, event records
// and cross-stream waits), which the host issues more slowly than the GPU runs them.  So
// the whole sequence is captured once into a HIP graph (on a private capture stream, the
// side streams joining through the same events) and replayed with one launch while the
// arguments stay the same; one graph is kept per host thread and device, rebuilt when
// any argument changes.  A caller's stream that is itself being captured gets the
// operations directly.
struct RGraph {
  int device = -1;
  hipStream_t cap = nullptr;
  hipGraphExec_t exec = nullptr;
  const float* H = nullptr;
  int64_t d = -1;
  const int32_t* perm = nullptr;
  float* Rt = nullptr;
  int64_t ldr = -1;
  void* ws = nullptr;
  uint32_t* flag = nullptr;
};

RGraph* rgraph() {
  thread_local std::vector<RGraph> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  for (RGraph& g : cache)
    if (g.device == dev) return g.cap ? &g : nullptr;
  RGraph g;
  g.device = dev;
  if (hipStreamCreateWithFlags(&g.cap, hipStreamNonBlocking) != hipSuccess) g.cap = nullptr;
  cache.push_back(g);
  return cache.back().cap ? &cache.back() : nullptr;
}

}  // namespace

int rfactor(const float* H, int64_t d, const int32_t* perm, float* Rt, int64_t ldr, void* ws,
            uint32_t* flag, hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) st = hipStreamCaptureStatusActive;
  RGraph* g = (st == hipStreamCaptureStatusNone && lookahead()) ? rgraph() : nullptr;
  if (!g) return rfactor_enqueue(H, d, perm, Rt, ldr, ws, flag, s);
  const bool same = g->exec && g->H == H && g->d == d && g->perm == perm && g->Rt == Rt &&
                    g->ldr == ldr && g->ws == ws && g->flag == flag;
  if (!same) {
    if (g->exec) {
      QZ_HIP(hipGraphExecDestroy(g->exec));
      g->exec = nullptr;
    }
    QZ_HIP(hipStreamBeginCapture(g->cap, hipStreamCaptureModeThreadLocal));
    const int rc = rfactor_enqueue(H, d, perm, Rt, ldr, ws, flag, g->cap);
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(g->cap, &graph);
    if (rc != QZ_OK || e != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      return rc != QZ_OK ? rc : fail(QZ_EHIP, "rfactor: graph capture failed");
    }
    const hipError_t ei = hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) {
      g->exec = nullptr;
      return fail(QZ_EHIP, "rfactor: graph instantiation failed");
    }
    g->H = H; g->d = d; g->perm = perm; g->Rt = Rt; g->ldr = ldr; g->ws = ws; g->flag = flag;
  }
  QZ_HIP(hipGraphLaunch(g->exec, s));
  return QZ_OK;
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
