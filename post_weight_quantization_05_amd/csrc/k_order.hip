// Quantization orders and the no-clip error bound (Babai page, technical summary, 2.3:
// without clipping a row's error is bounded by a quarter of its squared scales weighted
// by the diagonal D of the LDL factorisation of the reordered Hessian (Theorem 5); the
// bound depends on the order; a min-pivot order, taking the smallest remaining diagonal
// entry at every LDL step, keeps the trace of D small, and act order (descending
// Hessian diagonal) approximates it cheaply).
//
// The nearest-plane recursion eliminates coordinates in the reverse of the quantization
// order, so the min-pivot order here is the reverse of the elimination order of a
// pivoted LDL that takes, at each step, the smallest Schur-complement diagonal (among
// equal pivots the larger original index first, so that ties go to the smaller index in
// quantization order, as in act order).
//
// Pivoted LDL (fp64, blocked like a pivoted Cholesky): the full symmetric matrix A is
// kept; panels of PW columns are factored by one workgroup, left-looking inside the
// panel (column k = row k of the symmetric trailing matrix minus the panel's earlier
// columns), with the current Schur diagonal kept in `dcur` for the argmin; a chosen
// pivot is swapped into place (rows and columns of the trailing square, the panel's
// entries, dcur and the index map); after a panel the trailing square is updated with
// the panel's columns (tile products, both triangles, so it stays exactly symmetric)
// and dcur is refreshed from its diagonal.
#include "qz_internal.h"

namespace qz {

namespace {

constexpr int kThreads = 256;
constexpr int PW = 32;          // panel width
constexpr int PT = 1024;        // panel workgroup
constexpr int TT = 64;          // trailing tile

// ------------------------------------------------------------------ act order
__global__ void diag_kernel(const float* __restrict__ H, int64_t d, float* __restrict__ dg,
                            uint32_t* __restrict__ flag) {
  const int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (j >= d) return;
  const float v = H[j * d + j];
  if (!__builtin_isfinite(v)) atomicOr(flag, FLAG_NONFINITE);
  dg[j] = v;
}

// rank of j = #{i : dg_i > dg_j, or dg_i == dg_j and i < j}; perm[rank] = j.  The
// diagonal is staged through LDS in chunks.
__global__ __launch_bounds__(kThreads) void act_rank_kernel(const float* __restrict__ dg,
                                                            int64_t d, int32_t* __restrict__ perm) {
  constexpr int CH = 2048;
  __shared__ float tile[CH];
  const int64_t j = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  const float hj = j < d ? dg[j] : 0.f;
  int64_t rank = 0;
  for (int64_t base = 0; base < d; base += CH) {
    const int64_t lim = (d - base) < CH ? (d - base) : CH;
    for (int e = threadIdx.x; e < lim; e += kThreads) tile[e] = dg[base + e];
    __syncthreads();
    for (int t = 0; t < lim; ++t) {
      const float hi = tile[t];
      const int64_t i = base + t;
      rank += (hi > hj) || (hi == hj && i < j);
    }
    __syncthreads();
  }
  if (j < d) perm[rank] = static_cast<int32_t>(j);
}

// ------------------------------------------------------------------ min-pivot order
__global__ __launch_bounds__(kThreads) void mp_init(const float* __restrict__ H, int64_t n,
                                                    double* __restrict__ A,
                                                    double* __restrict__ dcur,
                                                    int32_t* __restrict__ idx,
                                                    uint32_t* __restrict__ flag) {
  bool bad = false;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n * n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const float h = H[e];
    bad |= !__builtin_isfinite(h);
    A[e] = static_cast<double>(h);
    const int64_t i = e / n;
    if (e == i * n + i) {
      dcur[i] = static_cast<double>(h);
      idx[i] = static_cast<int32_t>(i);
    }
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, FLAG_NONFINITE);
}

__device__ __forceinline__ bool mp_better(double d, int p, double bd, int bp) {
  return d < bd || (d == bd && p > bp);   // smallest pivot; ties: larger original index
}

// Steps k0 .. k1-1 of the elimination.  P[c][i] (c < PW, row-major [PW x n]) holds
// column k0 + c of L (its entries below the diagonal; the diagonal itself is not kept).
__global__ __launch_bounds__(PT) void mp_panel(const float* __restrict__ H, double* __restrict__ A,
                                               int64_t n, int64_t k0, int64_t k1,
                                               double* __restrict__ dcur,
                                               int32_t* __restrict__ idx,
                                               double* __restrict__ piv, double* __restrict__ P,
                                               uint32_t* __restrict__ flag) {
  __shared__ double rd[PT / 64];
  __shared__ int64_t ri[PT / 64];
  __shared__ int rp[PT / 64];
  __shared__ double pk[PW];
  __shared__ int64_t s_best;
  __shared__ double s_pv;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  for (int64_t k = k0; k < k1; ++k) {
    const int kk = static_cast<int>(k - k0);
    double bd = __builtin_inf();
    int64_t bi = -1;
    int bp = -1;
    for (int64_t i = k + tid; i < n; i += PT) {
      const double d = dcur[i];
      const int p = idx[i];
      if (mp_better(d, p, bd, bp)) { bd = d; bi = i; bp = p; }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const double od = __shfl_xor(bd, off);
      const int64_t oi = __shfl_xor(bi, off);
      const int op = __shfl_xor(bp, off);
      if (oi >= 0 && (bi < 0 || mp_better(od, op, bd, bp))) { bd = od; bi = oi; bp = op; }
    }
    if (lane == 0) { rd[wid] = bd; ri[wid] = bi; rp[wid] = bp; }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < PT / 64; ++w)
        if (ri[w] >= 0 && (bi < 0 || mp_better(rd[w], rp[w], bd, bp))) { bd = rd[w]; bi = ri[w]; bp = rp[w]; }
      s_best = bi;
      s_pv = bd;
    }
    __syncthreads();
    const int64_t js = s_best;
    const double pv = s_pv;
    // a pivot <= 1e-12 of its column's original diagonal (or none finite): not PD
    const bool bad = js < 0 || !(pv > 1e-12 * static_cast<double>(H[static_cast<int64_t>(idx[js]) * n + idx[js]]));
    if (bad) {
      if (tid == 0) atomicOr(flag, FLAG_NOTPD);
      return;   // uniform: every thread read the same s_best / s_pv
    }
    if (js != k) {
      for (int64_t c = k + tid; c < n; c += PT) {
        const double t = A[k * n + c];
        A[k * n + c] = A[js * n + c];
        A[js * n + c] = t;
      }
      __syncthreads();
      for (int64_t r = k + tid; r < n; r += PT) {
        const double t = A[r * n + k];
        A[r * n + k] = A[r * n + js];
        A[r * n + js] = t;
      }
      if (tid < kk) {
        const double t = P[tid * n + k];
        P[tid * n + k] = P[tid * n + js];
        P[tid * n + js] = t;
      }
      if (tid == 0) {
        const double td = dcur[k];
        dcur[k] = dcur[js];
        dcur[js] = td;
        const int32_t ti = idx[k];
        idx[k] = idx[js];
        idx[js] = ti;
      }
      __syncthreads();
    }
    if (tid == 0) piv[k] = pv;
    if (tid < kk) pk[tid] = P[tid * n + k];
    __syncthreads();
    const double inv = 1.0 / sqrt(pv);
    for (int64_t i = k + 1 + tid; i < n; i += PT) {
      double v = A[k * n + i];                 // = A[i][k]: the trailing square is symmetric
      for (int c = 0; c < kk; ++c) v -= P[c * n + i] * pk[c];
      const double l = v * inv;
      P[kk * n + i] = l;
      dcur[i] -= l * l;
    }
    __syncthreads();
  }
}

// A[i][j] -= sum_{c < w} P[c][i] P[c][j] for i, j >= k1 (both triangles, the same products
// in the same order, so the square stays exactly symmetric); dcur[i] = new A[i][i].
__global__ __launch_bounds__(kThreads) void mp_trailing(double* __restrict__ A, int64_t n,
                                                        int64_t k1, int w,
                                                        const double* __restrict__ P,
                                                        double* __restrict__ dcur) {
  __shared__ double Pi[PW][TT];
  __shared__ double Pj[PW][TT];
  const int64_t m = n - k1;
  const int64_t tiles = (m + TT - 1) / TT;
  const int64_t ti = blockIdx.x / tiles, tj = blockIdx.x % tiles;
  const int64_t i0 = k1 + ti * TT, j0 = k1 + tj * TT;
  const int tid = threadIdx.x;
  for (int e = tid; e < PW * TT; e += kThreads) {
    const int c = e / TT, t = e % TT;
    const bool okc = c < w;
    Pi[c][t] = (okc && i0 + t < n) ? P[c * n + i0 + t] : 0.0;
    Pj[c][t] = (okc && j0 + t < n) ? P[c * n + j0 + t] : 0.0;
  }
  __syncthreads();
  const int a0 = 4 * (tid / 16), b0 = 4 * (tid % 16);
  double acc[4][4] = {};
  for (int c = 0; c < w; ++c) {
    double x[4], y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) { x[u] = Pi[c][a0 + u]; y[u] = Pj[c][b0 + u]; }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = fma(x[u], y[v], acc[u][v]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i0 + a0 + u;
    if (i >= n) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t j = j0 + b0 + v;
      if (j >= n) continue;
      const double nv = A[i * n + j] - acc[u][v];
      A[i * n + j] = nv;
      if (i == j) dcur[i] = nv;
    }
  }
}

__global__ void mp_finish(const int32_t* __restrict__ idx, const double* __restrict__ piv,
                          int64_t n, int32_t* __restrict__ perm, double* __restrict__ pivots) {
  const int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (j >= n) return;
  perm[j] = idx[n - 1 - j];
  if (pivots) pivots[j] = piv[n - 1 - j];
}

// ------------------------------------------------------------------ error bound
// row_bound[r] = 1/8 sum_j D[j] s(r, perm[j] / group)^2, fixed-order fp64 reduction.
__global__ __launch_bounds__(kThreads) void bound_rows_kernel(const double* __restrict__ D,
                                                              const int32_t* __restrict__ perm,
                                                              const float* __restrict__ scales,
                                                              int64_t d_i, int group,
                                                              double* __restrict__ row_bound) {
  __shared__ double red[kThreads];
  const int64_t r = blockIdx.x;
  const int64_t G = d_i / group;
  double acc = 0.0;
  for (int64_t j = threadIdx.x; j < d_i; j += kThreads) {
    const int64_t col = perm ? perm[j] : j;
    const double s = static_cast<double>(scales[r * G + col / group]);
    acc += D[j] * s * s;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) row_bound[r] = 0.125 * red[0];
}

__global__ __launch_bounds__(kThreads) void sum_rows_kernel(const double* __restrict__ v, int64_t n,
                                                            double* __restrict__ total) {
  __shared__ double red[kThreads];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += kThreads) acc += v[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) *total = red[0];
}

inline unsigned blocks_for(int64_t n, int threads) {
  const int64_t b = (n + threads - 1) / threads;
  return static_cast<unsigned>(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

}  // namespace

size_t order_ws_bytes(int64_t n, int kind) {
  Carver c(nullptr);
  if (kind == QZ_ORDER_ACT) {
    c.take<float>(static_cast<size_t>(n));
    return c.used;
  }
  c.take<double>(static_cast<size_t>(n) * n);   // A
  c.take<double>(static_cast<size_t>(n));       // dcur
  c.take<int32_t>(static_cast<size_t>(n));      // idx
  c.take<double>(static_cast<size_t>(n));       // pivots in elimination order
  c.take<double>(static_cast<size_t>(PW) * n);  // panel
  return c.used;
}

int order_act(const float* H, int64_t n, int32_t* perm, void* ws, uint32_t* flag, hipStream_t s) {
  Carver cv(ws);
  float* dg = cv.take<float>(static_cast<size_t>(n));
  diag_kernel<<<blocks_for(n, kThreads), kThreads, 0, s>>>(H, n, dg, flag);
  QZ_TRY(check_launch("order.diag"));
  const int64_t nb = (n + kThreads - 1) / kThreads;
  if (nb > 0x7fffffff) return fail(QZ_EINVAL, "order: too many columns");
  act_rank_kernel<<<static_cast<unsigned>(nb), kThreads, 0, s>>>(dg, n, perm);
  return check_launch("order.act_rank");
}

int order_min_pivot(const float* H, int64_t n, int32_t* perm, double* pivots, void* ws,
                    uint32_t* flag, hipStream_t s) {
  Carver cv(ws);
  double* A = cv.take<double>(static_cast<size_t>(n) * n);
  double* dcur = cv.take<double>(static_cast<size_t>(n));
  int32_t* idx = cv.take<int32_t>(static_cast<size_t>(n));
  double* piv = cv.take<double>(static_cast<size_t>(n));
  double* P = cv.take<double>(static_cast<size_t>(PW) * n);
  mp_init<<<blocks_for(n * n, kThreads), kThreads, 0, s>>>(H, n, A, dcur, idx, flag);
  QZ_TRY(check_launch("order.mp_init"));
  for (int64_t k0 = 0; k0 < n; k0 += PW) {
    const int64_t k1 = (k0 + PW < n) ? k0 + PW : n;
    mp_panel<<<1, PT, 0, s>>>(H, A, n, k0, k1, dcur, idx, piv, P, flag);
    QZ_TRY(check_launch("order.mp_panel"));
    if (k1 < n) {
      const int64_t tiles = (n - k1 + TT - 1) / TT;
      if (tiles * tiles > 0x7fffffff) return fail(QZ_EINVAL, "order: too many tiles");
      mp_trailing<<<static_cast<unsigned>(tiles * tiles), kThreads, 0, s>>>(
          A, n, k1, static_cast<int>(k1 - k0), P, dcur);
      QZ_TRY(check_launch("order.mp_trailing"));
    }
  }
  mp_finish<<<blocks_for(n, kThreads), kThreads, 0, s>>>(idx, piv, n, perm, pivots);
  return check_launch("order.mp_finish");
}

int launch_error_bound(const double* D, const int32_t* perm, const float* scales, int64_t d_o,
                       int64_t d_i, int group, double* row_bound, double* total, hipStream_t s) {
  if (d_o > 0) {
    if (d_o > 0x7fffffff) return fail(QZ_EINVAL, "error bound: too many rows");
    bound_rows_kernel<<<static_cast<unsigned>(d_o), kThreads, 0, s>>>(D, perm, scales, d_i, group,
                                                                        row_bound);
    QZ_TRY(check_launch("error_bound.rows"));
  }
  sum_rows_kernel<<<1, kThreads, 0, s>>>(row_bound, d_o, total);
  return check_launch("error_bound.total");
}

}  // namespace qz
