// Pairwise-swap local search on the grid (ADMM-Q summary, methodology, 2. key
// algorithmic components, local search: discrete moves that swap values between input
// positions of an output channel and directly lower the reconstruction error, run in
// parallel on the GPU).
//
// Move set and acceptance (the pages give neither; the reading):
//  * inside one group (scale s): single moves c_j += a and pair moves (c_j += a,
//    c_k += b), j < k, a, b in {-1, +1}; codes stay in [0, 2^bits - 1].  With the
//    gradient g = H (q - w_hat) and d = a s, d' = b s the exact change of
//    f = 1/2 (q - w_hat)^T H (q - w_hat) is
//        d g_j + 1/2 d^2 H_jj  (+ d' g_k + 1/2 d'^2 H_kk + d d' H_jk for a pair);
//  * each group proposes its smallest change if negative (ties to the smallest
//    (j, k, a, b), singles as k = j, b = a, -1 before +1);
//  * proposals are accepted group by group in ascending order when their change plus
//    their exact interaction with the moves already accepted in the step stays negative;
//    the accepted moves are applied together, so f drops by the sum of those values.
//
// The gradient G = (Q - W_hat) H is formed once by the matrix-core GEMM and then kept up
// to date: a row whose step accepted moves d_p at positions p adds sum_p d_p H[p, :] to
// its gradient row (H symmetric), in the order the moves were accepted.  A row whose
// step accepted nothing is finished (its next step would propose and reject the same
// moves), so each step runs over the list of rows still active.  A step is the proposal
// scan (one wavefront per (active row, group)) and the accept pass (one wavefront per
// active row), which also applies the codes and updates the gradient row.
#include "qz_internal.h"

// No fused multiply-add contraction: the proposal scan and the recovery of the best
// pair's combo must evaluate the same values bit for bit.
#pragma clang fp contract(off)

namespace qz {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGroup = 128;   // two 64-lane slots of positions per wavefront

// Candidates are ranked by (change, index) with index = (j * group + k) * 4 + combo,
// combo = 2 * (a > 0) + (b > 0): the canonical order (j, k, a, b).
__device__ __forceinline__ bool better(float df, int idx, float bdf, int bidx) {
  return df < bdf || (df == bdf && idx < bidx);
}

// Per column c: the largest |H[c][k]| over the other columns k of c's group (the bound
// on the pair term used to skip positions in the proposal scan).
__global__ void ls_hmax_kernel(const float* __restrict__ H, int64_t d_i, int group,
                               float* __restrict__ hmax) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= d_i) return;
  const int64_t c0 = (c / group) * group;
  float m = 0.f;
  for (int k = 0; k < group; ++k)
    if (c0 + k != c) m = fmaxf(m, fabsf(H[c * d_i + c0 + k]));
  hmax[c] = m;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// The single-move terms of position j: u_lo = -s g_j + 1/2 s^2 H_jj (code - 1), u_hi =
// +s g_j + 1/2 s^2 H_jj (code + 1), +inf where the code would leave [0, maxq].
__device__ __forceinline__ void single_terms(float gj, float hjj, float cj, float s, float s2,
                                             float maxq, float& ulo, float& uhi) {
  const float inf = __builtin_inff();
  const float half = 0.5f * s2 * hjj;
  ulo = (cj - 1.f >= 0.f) ? (-s * gj + half) : inf;
  uhi = (cj + 1.f <= maxq) ? (s * gj + half) : inf;
}

// The four pair values of (j, k) with t = s^2 H_jk, combos (a, b) = (-,-), (-,+), (+,-), (+,+).
struct Pair4 {
  float v0, v1, v2, v3;
};
__device__ __forceinline__ Pair4 pair_values(float ulj, float uhj, float ulk, float uhk, float t) {
  Pair4 p;
  p.v0 = (ulj + ulk) + t;
  p.v1 = (ulj + uhk) - t;
  p.v2 = (uhj + ulk) - t;
  p.v3 = (uhj + uhk) + t;
  return p;
}

// One wavefront per (active row, group).  Lane l holds position k = l + 64 sl of slot sl
// (its single terms in registers) and is credited with every candidate whose larger
// position is k: the pairs (j, k), j < k, in ascending j, then the single move of k, i.e.
// ascending candidate index, so inside a slot only a strictly smaller change displaces
// the best.  The wavefront walks j uniformly (the row H[j, group] is one coalesced load;
// j's terms are lane broadcasts).  Only negative changes matter, and position j is
// skipped when fl(min(u_lo j, u_hi j) + min over the group of u) >= fl(s^2 hmax_j): by
// monotonicity of rounding every computed pair value of j is then >= 0 (or NaN), so
// skipping changes nothing.  The combo of a slot's best pair is recovered at the end by
// recomputing its four values with the same operations (contraction off) and taking the
// first equal to the best.
template <int NS>
__global__ __launch_bounds__(kThreads) void ls_propose_kernel(
    const float* __restrict__ Gm, int64_t ldg, const float* __restrict__ H, int64_t d_i,
    const float* __restrict__ hmax, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, int group, int bits, const int32_t* __restrict__ act,
    int64_t n_act, float* __restrict__ best_df, int32_t* __restrict__ best_idx) {
  const int lane = threadIdx.x & 63;
  const int64_t G = d_i / group;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (w >= n_act * G) return;   // whole wavefront; no workgroup barrier below
  const int64_t r = act[w / G];
  const int64_t gi = w % G;
  const int64_t c0 = gi * group;
  const float s = scales[r * G + gi];
  const float s2 = s * s;
  const float maxq = static_cast<float>((1 << bits) - 1);
  const float inf = __builtin_inff();
  const float* __restrict__ grow = Gm + r * ldg + c0;
  const uint8_t* __restrict__ crow = codes + r * d_i + c0;
  const float* __restrict__ hblk = H + c0 * d_i + c0;   // H[c0 + j][c0 + k] = hblk[j d_i + k]

  float ul[NS], uh[NS];
  bool kin[NS];
  float umin = inf;
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int k = lane + 64 * sl;
    kin[sl] = k < group;
    ul[sl] = inf;
    uh[sl] = inf;
    if (kin[sl])
      single_terms(grow[k], hblk[k * d_i + k], static_cast<float>(crow[k]), s, s2, maxq, ul[sl],
                   uh[sl]);
    umin = fminf(umin, fminf(ul[sl], uh[sl]));
  }
  for (int off = 32; off > 0; off >>= 1) umin = fminf(umin, __shfl_xor(umin, off));
  uint64_t keep[NS];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int j = lane + 64 * sl;
    bool k_j = false;
    if (kin[sl]) {
      const float lower = fminf(ul[sl], uh[sl]) + umin;
      const float tmax = s2 * hmax[c0 + j];
      k_j = !(lower >= tmax);
    }
    keep[sl] = __ballot(k_j);
  }

  float bdf[NS];
  int bj[NS];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    bdf[sl] = 0.f;
    bj[sl] = -1;
  }
#pragma unroll
  for (int sj = 0; sj < NS; ++sj) {
    uint64_t m = keep[sj];
    while (m) {
      const int bit = __builtin_ctzll(m);
      m &= m - 1;
      const int j = 64 * sj + bit;
      const float ulj = readlane_f(ul[sj], bit), uhj = readlane_f(uh[sj], bit);
      const float* __restrict__ hrow = hblk + static_cast<int64_t>(j) * d_i;
#pragma unroll
      for (int sl = sj; sl < NS; ++sl) {
        const int k = lane + 64 * sl;
        const bool valid = kin[sl] && k > j;
        const float t = s2 * (valid ? hrow[k] : 0.f);
        const Pair4 p = pair_values(ulj, uhj, ul[sl], uh[sl], t);
        const float v = fminf(fminf(p.v0, p.v1), fminf(p.v2, p.v3));
        if (valid && v < bdf[sl]) {
          bdf[sl] = v;
          bj[sl] = j;
        }
      }
    }
  }
  // singles last in each slot, then the combo of each slot's best
  float fdf = 0.f;
  int fidx = 0x7fffffff;
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int k = lane + 64 * sl;
    if (!kin[sl]) continue;
    const float v = fminf(ul[sl], uh[sl]);
    if (v < bdf[sl]) {
      bdf[sl] = v;
      bj[sl] = k;
    }
    if (bj[sl] < 0) continue;
    const int j = bj[sl];
    int combo;
    if (j == k) {
      combo = (ul[sl] == bdf[sl]) ? 0 : 3;
    } else {
      float ulj, uhj;
      single_terms(grow[j], hblk[static_cast<int64_t>(j) * d_i + j], static_cast<float>(crow[j]), s,
                   s2, maxq, ulj, uhj);
      const float t = s2 * hblk[static_cast<int64_t>(j) * d_i + k];
      const Pair4 p = pair_values(ulj, uhj, ul[sl], uh[sl], t);
      combo = (p.v0 == bdf[sl]) ? 0 : (p.v1 == bdf[sl]) ? 1 : (p.v2 == bdf[sl]) ? 2 : 3;
    }
    const int idx = (j * group + k) * 4 + combo;
    if (better(bdf[sl], idx, fdf, fidx)) {
      fdf = bdf[sl];
      fidx = idx;
    }
  }
  // wavefront argmin over the lanes, ties to the smaller index
  for (int off = 32; off > 0; off >>= 1) {
    const float odf = __shfl_xor(fdf, off);
    const int oidx = __shfl_xor(fidx, off);
    if (better(odf, oidx, fdf, fidx)) { fdf = odf; fidx = oidx; }
  }
  if (lane == 0) {
    const bool improves = fidx != 0x7fffffff;   // only negative changes were kept
    best_df[r * G + gi] = improves ? fdf : 0.f;
    best_idx[r * G + gi] = improves ? fidx : -1;
  }
}

struct Move {
  int64_t p0, p1;   // columns (p1 = -1 for a single)
  float d0, d1;     // value changes
};

__device__ __forceinline__ Move decode(int idx, int64_t c0, int group, float s) {
  const int combo = idx & 3;
  const int jk = idx >> 2;
  const int j = jk / group, k = jk % group;
  Move m;
  m.p0 = c0 + j;
  m.d0 = (combo & 2) ? s : -s;
  if (k == j) {
    m.p1 = -1;
    m.d1 = 0.f;
  } else {
    m.p1 = c0 + k;
    m.d1 = (combo & 1) ? s : -s;
  }
  return m;
}

__device__ __forceinline__ void axpy4(float4& g, float v, const float4 h) {
  g.x = fmaf(v, h.x, g.x);
  g.y = fmaf(v, h.y, g.y);
  g.z = fmaf(v, h.z, g.z);
  g.w = fmaf(v, h.w, g.w);
}

// One wavefront (one workgroup) per active row.  Decision: proposals in ascending group
// order; the interaction of a proposal with the moves already accepted is summed by the
// lanes (one accepted move each, in turn) and reduced in a fixed order, so the decision
// is uniform.  The accepted moves live in LDS (16 bytes each, at most one per group).
// Then the codes change by one step per moved position, the row joins the next step's
// list, and (when `update`) its gradient row gains sum_p d_p H[p, :].
template <bool VEC>
__global__ __launch_bounds__(64) void ls_accept_kernel(
    const float* __restrict__ H, int64_t d_i, uint8_t* __restrict__ codes,
    const float* __restrict__ scales, int group, const float* __restrict__ best_df,
    const int32_t* __restrict__ best_idx, const int32_t* __restrict__ act,
    float* __restrict__ Gm, int64_t ldg, int update, int32_t* __restrict__ next_act,
    int32_t* __restrict__ counters) {
  extern __shared__ __attribute__((aligned(16))) unsigned char ls_smem[];
  int32_t* pos = reinterpret_cast<int32_t*>(ls_smem);                 // [2 * G]
  const int64_t G = d_i / group;
  float* val = reinterpret_cast<float*>(ls_smem + 8 * G);             // [2 * G]
  const int lane = threadIdx.x;
  const int64_t r = act[blockIdx.x];
  int n_acc = 0;
  for (int64_t gi = 0; gi < G; ++gi) {
    const int idx = best_idx[r * G + gi];
    if (idx < 0) continue;
    const Move m = decode(idx, gi * group, group, scales[r * G + gi]);
    float part = 0.f;
    for (int a = lane; a < n_acc; a += 64) {
      const int64_t q0 = pos[2 * a], q1 = pos[2 * a + 1];
      const float e0 = val[2 * a], e1 = val[2 * a + 1];
      float c = m.d0 * e0 * H[m.p0 * d_i + q0];
      if (q1 >= 0) c += m.d0 * e1 * H[m.p0 * d_i + q1];
      if (m.p1 >= 0) {
        c += m.d1 * e0 * H[m.p1 * d_i + q0];
        if (q1 >= 0) c += m.d1 * e1 * H[m.p1 * d_i + q1];
      }
      part += c;
    }
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    const float run = best_df[r * G + gi] + part;
    if (run < 0.f) {
      if (lane == 0) {
        pos[2 * n_acc] = static_cast<int32_t>(m.p0);
        pos[2 * n_acc + 1] = static_cast<int32_t>(m.p1);
        val[2 * n_acc] = m.d0;
        val[2 * n_acc + 1] = m.d1;
      }
      ++n_acc;
      __syncthreads();   // one wavefront: waits for the LDS writes
    }
  }
  if (n_acc == 0) return;
  uint8_t* row = codes + r * d_i;
  for (int a = lane; a < n_acc; a += 64) {
    const int32_t q0 = pos[2 * a], q1 = pos[2 * a + 1];
    row[q0] = static_cast<uint8_t>(static_cast<int>(row[q0]) + (val[2 * a] > 0.f ? 1 : -1));
    if (q1 >= 0)
      row[q1] = static_cast<uint8_t>(static_cast<int>(row[q1]) + (val[2 * a + 1] > 0.f ? 1 : -1));
  }
  if (lane == 0) {
    atomicAdd(&counters[0], n_acc);
    const int32_t slot = atomicAdd(&counters[1], 1);
    next_act[slot] = static_cast<int32_t>(r);
  }
  if (!update) return;
  float* __restrict__ grow = Gm + r * ldg;
  if constexpr (VEC) {
    // d_i % 4 == 0: lane l holds columns 4 (l + 64 u) .. +3 of each 1024-column chunk
    constexpr int U = 4;
    for (int64_t cb = 0; cb < d_i; cb += 256 * U) {
      float4 g[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t col = cb + 4 * (lane + 64 * u);
        g[u] = col < d_i ? *reinterpret_cast<const float4*>(grow + col) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      for (int t = 0; t < 2 * n_acc; ++t) {
        const int32_t p = pos[t];
        if (p < 0) continue;
        const float v = val[t];
        const float* __restrict__ hr = H + static_cast<int64_t>(p) * d_i;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t col = cb + 4 * (lane + 64 * u);
          if (col < d_i) axpy4(g[u], v, *reinterpret_cast<const float4*>(hr + col));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t col = cb + 4 * (lane + 64 * u);
        if (col < d_i) *reinterpret_cast<float4*>(grow + col) = g[u];
      }
    }
  } else {
    constexpr int U = 8;
    for (int64_t cb = 0; cb < d_i; cb += 64 * U) {
      float g[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t col = cb + lane + 64 * u;
        g[u] = col < d_i ? grow[col] : 0.f;
      }
      for (int t = 0; t < 2 * n_acc; ++t) {
        const int32_t p = pos[t];
        if (p < 0) continue;
        const float v = val[t];
        const float* __restrict__ hr = H + static_cast<int64_t>(p) * d_i;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t col = cb + lane + 64 * u;
          if (col < d_i) g[u] = fmaf(v, hr[col], g[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t col = cb + lane + 64 * u;
        if (col < d_i) grow[col] = g[u];
      }
    }
  }
}

__global__ void ls_iota_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = static_cast<int32_t>(i);
}

}  // namespace

int ls_max_group() { return kMaxGroup; }

int launch_ls_iota(int32_t* p, int64_t n, hipStream_t s) {
  if (n == 0) return QZ_OK;
  const int64_t nb = ceil_div(n, int64_t{256});
  if (nb > 0x7fffffff) return fail(QZ_EINVAL, "local search: too many rows");
  ls_iota_kernel<<<static_cast<unsigned>(nb), 256, 0, s>>>(p, n);
  return check_launch("ls_iota");
}

int launch_ls_hmax(const float* H, int64_t d_i, int group, float* hmax, hipStream_t s) {
  const int64_t nb = ceil_div(d_i, int64_t{256});
  if (nb > 0x7fffffff) return fail(QZ_EINVAL, "local search: too many columns");
  ls_hmax_kernel<<<static_cast<unsigned>(nb), 256, 0, s>>>(H, d_i, group, hmax);
  return check_launch("ls_hmax");
}

int launch_ls_propose(const float* Gm, int64_t ldg, const float* H, int64_t d_i,
                      const float* hmax, const uint8_t* codes, const float* scales, int group,
                      int bits, const int32_t* act, int64_t n_act, float* best_df,
                      int32_t* best_idx, hipStream_t s) {
  const int64_t waves = n_act * (d_i / group);
  if (waves == 0) return QZ_OK;
  const int64_t nb = ceil_div(waves, int64_t{kThreads / 64});
  if (nb > 0x7fffffff) return fail(QZ_EINVAL, "local search: too many groups");
  if (group <= 64)
    ls_propose_kernel<1><<<static_cast<unsigned>(nb), kThreads, 0, s>>>(
        Gm, ldg, H, d_i, hmax, codes, scales, group, bits, act, n_act, best_df, best_idx);
  else
    ls_propose_kernel<2><<<static_cast<unsigned>(nb), kThreads, 0, s>>>(
        Gm, ldg, H, d_i, hmax, codes, scales, group, bits, act, n_act, best_df, best_idx);
  return check_launch("ls_propose");
}

size_t ls_accept_lds(int64_t G) { return static_cast<size_t>(G) * 16; }

int launch_ls_accept(const float* H, int64_t d_i, uint8_t* codes, const float* scales, int group,
                     const float* best_df, const int32_t* best_idx, const int32_t* act,
                     int64_t n_act, float* Gm, int64_t ldg, bool update, int32_t* next_act,
                     int32_t* counters, hipStream_t s) {
  if (n_act == 0) return QZ_OK;
  if (n_act > 0x7fffffff) return fail(QZ_EINVAL, "local search: too many rows");
  const size_t lds = ls_accept_lds(d_i / group);
  const bool vec = (d_i % 4 == 0) && (ldg % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(H) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(Gm) % 16 == 0);
  if (vec)
    ls_accept_kernel<true><<<static_cast<unsigned>(n_act), 64, lds, s>>>(
        H, d_i, codes, scales, group, best_df, best_idx, act, Gm, ldg, update ? 1 : 0, next_act,
        counters);
  else
    ls_accept_kernel<false><<<static_cast<unsigned>(n_act), 64, lds, s>>>(
        H, d_i, codes, scales, group, best_df, best_idx, act, Gm, ldg, update ? 1 : 0, next_act,
        counters);
  return check_launch("ls_accept");
}

}  // namespace qz
