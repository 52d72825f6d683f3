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
// A step is: gradient G = (Q - W_hat) H (the GEMM, fp32), the proposal scan (one
// wavefront per (row, group)), the accept pass (one wavefront per row).
#include "qz_internal.h"

namespace qz {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGroup = 128;

// Candidates are ranked by (change, index) with index = (j * group + k) * 4 + combo,
// combo = 2 * (a > 0) + (b > 0): the canonical order (j, k, a, b).
__device__ __forceinline__ bool better(float df, int idx, float bdf, int bidx) {
  return df < bdf || (df == bdf && idx < bidx);
}

// One wavefront per (row, group).  Lane l (< group / 2) owns positions l and
// group - 1 - l and scans their partners above them, so every lane does group - 1
// pair evaluations.
__global__ __launch_bounds__(kThreads) void ls_propose_kernel(
    const float* __restrict__ Gm, int64_t ldg, const float* __restrict__ H, int64_t d_i,
    const uint8_t* __restrict__ codes, const float* __restrict__ scales, int64_t d_o, int group,
    int bits, float* __restrict__ best_df, int32_t* __restrict__ best_idx) {
  __shared__ float u_lo[kThreads / 64][kMaxGroup];
  __shared__ float u_hi[kThreads / 64][kMaxGroup];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int64_t G = d_i / group;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wid;
  const bool live = w < d_o * G;
  const int64_t r = live ? w / G : 0;
  const int64_t gi = live ? w % G : 0;
  const int64_t c0 = gi * group;
  const float s = live ? scales[r * G + gi] : 0.f;
  const float s2 = s * s;
  const float maxq = static_cast<float>((1 << bits) - 1);
  const float inf = __builtin_inff();
  if (live) {
    for (int j = lane; j < group; j += 64) {
      const float gj = Gm[r * ldg + c0 + j];
      const float hjj = H[(c0 + j) * d_i + c0 + j];
      const float cj = static_cast<float>(codes[r * d_i + c0 + j]);
      const float half = 0.5f * s2 * hjj;
      u_lo[wid][j] = (cj - 1.f >= 0.f) ? (-s * gj + half) : inf;
      u_hi[wid][j] = (cj + 1.f <= maxq) ? (s * gj + half) : inf;
    }
  }
  __syncthreads();
  float bdf = inf;
  int bidx = 0x7fffffff;
  if (live && lane < group / 2 + (group & 1)) {
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      const int j = h == 0 ? lane : group - 1 - lane;
      if (h == 1 && j <= lane) break;
      const float ulj = u_lo[wid][j], uhj = u_hi[wid][j];
      // singles
      {
        const int base = (j * group + j) * 4;
        if (better(ulj, base + 0, bdf, bidx)) { bdf = ulj; bidx = base + 0; }
        if (better(uhj, base + 3, bdf, bidx)) { bdf = uhj; bidx = base + 3; }
      }
      const float* __restrict__ hrow = H + (c0 + j) * d_i + c0;
      for (int k = j + 1; k < group; ++k) {
        const float t = s2 * hrow[k];
        const float ulk = u_lo[wid][k], uhk = u_hi[wid][k];
        const int base = (j * group + k) * 4;
        const float v0 = ulj + ulk + t;    // (-1, -1)
        const float v1 = ulj + uhk - t;    // (-1, +1)
        const float v2 = uhj + ulk - t;    // (+1, -1)
        const float v3 = uhj + uhk + t;    // (+1, +1)
        if (better(v0, base + 0, bdf, bidx)) { bdf = v0; bidx = base + 0; }
        if (better(v1, base + 1, bdf, bidx)) { bdf = v1; bidx = base + 1; }
        if (better(v2, base + 2, bdf, bidx)) { bdf = v2; bidx = base + 2; }
        if (better(v3, base + 3, bdf, bidx)) { bdf = v3; bidx = base + 3; }
      }
    }
  }
  // wavefront argmin, same order
  for (int off = 32; off > 0; off >>= 1) {
    const float odf = __shfl_xor(bdf, off);
    const int oidx = __shfl_xor(bidx, off);
    if (better(odf, oidx, bdf, bidx)) { bdf = odf; bidx = oidx; }
  }
  if (live && lane == 0) {
    const bool improves = bdf < 0.f;   // NaN and +inf propose nothing
    best_df[w] = improves ? bdf : 0.f;
    best_idx[w] = improves ? bidx : -1;
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

// One wavefront (one workgroup) per row: proposals in ascending group order; the
// interaction of a proposal with the moves already accepted is summed by the lanes (one
// accepted move each, in turn) and reduced in a fixed order, so the decision is uniform.
// The accepted moves live in LDS (16 bytes each, at most one per group).
__global__ __launch_bounds__(64) void ls_accept_kernel(
    const float* __restrict__ H, int64_t d_i, uint8_t* __restrict__ codes,
    const float* __restrict__ scales, int64_t d_o, int group, const float* __restrict__ best_df,
    const int32_t* __restrict__ best_idx, int32_t* __restrict__ counter) {
  extern __shared__ __attribute__((aligned(16))) unsigned char ls_smem[];
  int32_t* pos = reinterpret_cast<int32_t*>(ls_smem);                 // [2 * G]
  const int64_t G = d_i / group;
  float* val = reinterpret_cast<float*>(ls_smem + 8 * G);             // [2 * G]
  const int lane = threadIdx.x;
  const int64_t r = blockIdx.x;
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
  // apply: each accepted move changes its codes by one step
  uint8_t* row = codes + r * d_i;
  for (int a = lane; a < n_acc; a += 64) {
    const int32_t q0 = pos[2 * a], q1 = pos[2 * a + 1];
    row[q0] = static_cast<uint8_t>(static_cast<int>(row[q0]) + (val[2 * a] > 0.f ? 1 : -1));
    if (q1 >= 0)
      row[q1] = static_cast<uint8_t>(static_cast<int>(row[q1]) + (val[2 * a + 1] > 0.f ? 1 : -1));
  }
  if (lane == 0 && n_acc > 0) atomicAdd(counter, n_acc);
}

}  // namespace

int ls_max_group() { return kMaxGroup; }

int launch_ls_propose(const float* Gm, int64_t ldg, const float* H, int64_t d_i,
                      const uint8_t* codes, const float* scales, int64_t d_o, int group, int bits,
                      float* best_df, int32_t* best_idx, hipStream_t s) {
  const int64_t waves = d_o * (d_i / group);
  if (waves == 0) return QZ_OK;
  const int64_t nb = ceil_div(waves, int64_t{kThreads / 64});
  if (nb > 0x7fffffff) return fail(QZ_EINVAL, "local search: too many groups");
  ls_propose_kernel<<<static_cast<unsigned>(nb), kThreads, 0, s>>>(Gm, ldg, H, d_i, codes, scales,
                                                                    d_o, group, bits, best_df,
                                                                    best_idx);
  return check_launch("ls_propose");
}

size_t ls_accept_lds(int64_t G) { return static_cast<size_t>(G) * 16; }

int launch_ls_accept(const float* H, int64_t d_i, uint8_t* codes, const float* scales,
                     int64_t d_o, int group, const float* best_df, const int32_t* best_idx,
                     int32_t* counter, hipStream_t s) {
  if (d_o == 0) return QZ_OK;
  if (d_o > 0x7fffffff) return fail(QZ_EINVAL, "local search: too many rows");
  const size_t lds = ls_accept_lds(d_i / group);
  ls_accept_kernel<<<static_cast<unsigned>(d_o), 64, lds, s>>>(H, d_i, codes, scales, d_o, group,
                                                                best_df, best_idx, counter);
  return check_launch("ls_accept");
}

}  // namespace qz
