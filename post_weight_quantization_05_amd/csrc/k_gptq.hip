// GPTQ in-block column kernel (GPTQ tutorial, section 3: the column-by-column part of
// the blocked quantizer; section 2 gives the compensation it applies).  Inside a block
// of at most 128 columns the columns are fixed one after another in the common order:
// every row rounds its current value of the column on its static grid, and the error
// divided by the pivot R_jj (kept per row as the block's E) is passed on to the block's
// remaining columns along row j of R.  Columns after the block receive all of the
// block's errors at once, through the separate matrix-core product in k_gemm.hip.
//
// The rows are independent (they share only R), so a workgroup owns 16 rows and steps
// through the columns for all of them together.  The 16 lanes of a DPP row share one
// weight row; lane l keeps columns l, l+16, ..., l+112 of the block in registers, with
// its row's (scale, zero) for each of them, so neither the block of W nor the grid
// passes through LDS.  At step j the lane holding column j rounds it (the correctly
// rounded fp32 quotient, half-to-even) and forms the scaled error, a DPP row broadcast
// (row_newbcast) hands it to the other fifteen lanes, and each lane updates its later
// columns with its eight entries of R's row j, read from LDS as two 16-byte vectors.
// The workgroup's set-up stages R's block with many global loads in flight (clamped
// addresses, selected afterwards); at the end each lane writes E and the codes of its
// columns.  Small workgroups (16 rows, about 68 KB of LDS) keep every CU busy from 4096
// rows up.
#include "qz_internal.h"

namespace qz {

namespace {

constexpr int MAXB = 128;               // largest block
constexpr int LPR = 16;                 // lanes per row: one DPP row
constexpr int PER = MAXB / LPR;         // columns per lane: l, l + 16, ..., l + 112
constexpr int RJ = MAXB + 4;            // LDS stride of an R row, floats (16-byte aligned rows)

// Lane O of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int O>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + O, 0xF, 0xF, false));
}

// The correctly rounded quotient x / s from y = RN(1 / s), formed once per column: with
// q0 = RN(x y) within an ulp of x / s, the remainder x - s q0 is exact in one FMA and
// RN(q0 + r y) is RN(x / s) (Markstein's theorem on division by a correctly rounded
// reciprocal), so the codes are those of the IEEE division at three operations instead of
// the eleven of the full division sequence on the step's dependency chain.  (Values whose
// quotient or remainder leaves the normal range only reach codes that the rounding and
// the clamp make the same.)
__device__ __forceinline__ float div_rn(float x, float s, float y) {
  const float q0 = x * y;
  const float r = __builtin_fmaf(-s, q0, x);
  return __builtin_fmaf(r, y, q0);
}

// Clamped and unclamped (kept inside the int32 range) codes rint(x / s) + z.
__device__ __forceinline__ float code_of(float q, float z, float maxq) {
  return fminf(fmaxf(__builtin_rintf(q) + z, 0.0f), maxq);
}
__device__ __forceinline__ float code_of_noclip(float q, float z) {
  return fminf(fmaxf(__builtin_rintf(q) + z, -2147483648.0f), 2147483520.0f);
}

// Entries l + 16 i of R's row j and 1 / R_jj, read from LDS one step ahead.
struct RRow {
  float v[PER];
  float rinv;
};
__device__ __forceinline__ void load_rrow(RRow& r, const float* Rb, const float* rinv, int j, int l) {
  const float4* rr = reinterpret_cast<const float4*>(Rb + j * RJ + l * PER);
  const float4 r0 = rr[0], r1 = rr[1];
  r.v[0] = r0.x; r.v[1] = r0.y; r.v[2] = r0.z; r.v[3] = r0.w;
  r.v[4] = r1.x; r.v[5] = r1.y; r.v[6] = r1.z; r.v[7] = r1.w;
  r.rinv = rinv[j];
}

template <int J, bool NOCLIP>
__device__ __forceinline__ void column_step(float (&wr)[PER], float (&cr)[PER], const float (&sv)[PER],
                                            const float (&yv)[PER], const float (&zv)[PER],
                                            float maxq, const RRow& r, int l) {
  constexpr int owner = J % LPR, slot = J / LPR;
  // every lane rounds its own value of slot `slot`; only the owner's is used
  const float x = wr[slot];
  const float q = div_rn(x, sv[slot], yv[slot]);
  const float c = NOCLIP ? code_of_noclip(q, zv[slot]) : code_of(q, zv[slot], maxq);
  const float qv = sv[slot] * (c - zv[slot]);
  const float err = (x - qv) * r.rinv;
  const bool own = (l == owner);
  wr[slot] = own ? err : x;
  cr[slot] = own ? c : cr[slot];
  const float e = row_bcast<owner>(err);
  // the later columns of the block get E R[j, col]; in slot `slot` those are the lanes
  // after the owner (the others hold finished columns and subtract zero)
  const float es = (l > owner) ? e : 0.f;
  wr[slot] -= es * r.v[slot];
#pragma unroll
  for (int i = slot + 1; i < PER; ++i) wr[i] -= e * r.v[i];
}

template <int J, bool NOCLIP>
struct Steps {
  __device__ static __forceinline__ void run(int w, float (&wr)[PER], float (&cr)[PER],
                                             const float (&sv)[PER], const float (&yv)[PER],
                                             const float (&zv)[PER], float maxq, const float* Rb,
                                             const float* rinv, const RRow& cur, int l) {
    if (J >= w) return;   // uniform: blocks narrower than MAXB stop early
    RRow next;
    if (J + 1 < MAXB) load_rrow(next, Rb, rinv, J + 1 < MAXB ? J + 1 : J, l);
    column_step<J, NOCLIP>(wr, cr, sv, yv, zv, maxq, cur, l);
    // one step's work per scheduling region: the next row's reads issue before it
    __builtin_amdgcn_sched_barrier(0);
    Steps<J + 1, NOCLIP>::run(w, wr, cr, sv, yv, zv, maxq, Rb, rinv, next, l);
  }
};
template <bool NOCLIP>
struct Steps<MAXB, NOCLIP> {
  __device__ static __forceinline__ void run(int, float (&)[PER], float (&)[PER], const float (&)[PER],
                                             const float (&)[PER], const float (&)[PER], float,
                                             const float*, const float*, const RRow&, int) {}
};

// NOCLIP: codes are not clamped to [0, 2^b - 1] (the Babai page's no-clipping regime)
// and are written as int32 to codes32.
template <bool NOCLIP, int ROWS>
__global__ __launch_bounds__(ROWS * LPR) void gptq_block_kernel(
    float* __restrict__ W, int64_t ldw, int64_t d_o, int64_t a, int w,
    const float* __restrict__ Rt, int64_t ldr, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int64_t G, int group, float maxq,
    const int32_t* __restrict__ perm, float* __restrict__ E, int64_t lde,
    uint8_t* __restrict__ codes, int32_t* __restrict__ codes32, int64_t d_i) {
  // R[a+j][a+l+16i] at Rb[j * RJ + l * PER + i]: lane l reads its 8 entries of row j with
  // two 16-byte LDS reads, and the 16 lanes of a row read 128 consecutive floats
  __shared__ __attribute__((aligned(16))) float Rb[MAXB * RJ];
  __shared__ float rinv[MAXB];

  const int tid = threadIdx.x;
  const int l = tid % LPR;
  const int rl = tid / LPR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * ROWS + rl;
  const bool rok = row < d_o;
  const int64_t crow = rok ? row : d_o - 1;   // clamped row for the grid loads

  constexpr int kThreads = ROWS * LPR;
  // R block (upper part, c >= j) into LDS.  Loads are issued 16 at a time from clamped
  // (always valid) addresses and selected afterwards, so their latencies overlap; each
  // wavefront reads 64 consecutive entries of one row of Rt.
  {
    constexpr int RIT = MAXB * MAXB / kThreads;
    constexpr int RU = 16;
#pragma unroll
    for (int it0 = 0; it0 < RIT; it0 += RU) {
      float v[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int e = tid + (it0 + u) * kThreads;
        const int c = e / MAXB, j = e % MAXB;
        const int cc = c < w ? c : w - 1, jj = j < w ? j : w - 1;
        const float x = Rt[(a + cc) * ldr + a + jj];
        v[u] = (c < w && j < w && c >= j) ? x : 0.f;
      }
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int e = tid + (it0 + u) * kThreads;
        const int c = e / MAXB, j = e % MAXB;
        Rb[j * RJ + (c % LPR) * PER + c / LPR] = v[u];
      }
    }
  }
  for (int j = tid; j < w; j += kThreads) rinv[j] = 1.0f / Rt[(a + j) * ldr + a + j];

  // the row's block of W and, per owned column, the row's grid (groups are ranges of
  // ORIGINAL columns)
  float wr[PER], sv[PER], yv[PER], zv[PER], cr[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = l + LPR * i;
    const int cc = c < w ? c : w - 1;
    const int64_t oc = perm ? perm[a + cc] : a + cc;
    const int64_t gi = crow * G + oc / group;
    sv[i] = scales[gi];
    yv[i] = 1.0f / sv[i];   // IEEE division: the correctly rounded reciprocal
    zv[i] = static_cast<float>(zeros[gi]);
    wr[i] = (rok && c < w) ? W[row * ldw + a + c] : 0.f;
    cr[i] = 0.f;
  }
  __syncthreads();

  RRow first;
  load_rrow(first, Rb, rinv, 0, l);
  Steps<0, NOCLIP>::run(w, wr, cr, sv, yv, zv, maxq, Rb, rinv, first, l);

  // E (the scaled errors, for the matrix-core update of the later columns) and the codes;
  // for each slot the 16 lanes of a row write 16 consecutive columns
  if (rok) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = l + LPR * i;
      if (c >= w) continue;
      E[row * lde + c] = wr[i];
      const int64_t oc = perm ? perm[a + c] : a + c;
      if constexpr (NOCLIP)
        codes32[row * d_i + oc] = static_cast<int32_t>(cr[i]);
      else
        codes[row * d_i + oc] = static_cast<uint8_t>(cr[i]);
    }
  }
}

}  // namespace

int launch_gptq_block(float* W, int64_t ldw, int64_t d_o, int64_t a, int64_t b, const float* Rt,
                      int64_t ldr, const float* scales, const uint8_t* zeros, int64_t n_groups,
                      int group, int bits, const int32_t* perm, float* E, int64_t lde,
                      uint8_t* codes, int32_t* codes32, int64_t d_i, hipStream_t s) {
  const int w = static_cast<int>(b - a);
  if (w <= 0 || w > MAXB) return fail(QZ_EINVAL, "gptq block width out of range");
  if (!codes == !codes32) return fail(QZ_EINVAL, "gptq block: exactly one code output");
  const float maxq = static_cast<float>((1 << bits) - 1);
  // 16 rows per workgroup up to 8192 rows (every CU busy from 4096 rows up), 32 above (one
  // round of resident workgroups at 12288 rows)
  const bool tall = d_o > 8192;
  const unsigned nb = static_cast<unsigned>(ceil_div(d_o, tall ? 32 : 16));
  if (codes32) {
    if (tall)
      gptq_block_kernel<true, 32><<<nb, 32 * LPR, 0, s>>>(W, ldw, d_o, a, w, Rt, ldr, scales, zeros,
                                                          n_groups, group, maxq, perm, E, lde,
                                                          nullptr, codes32, d_i);
    else
      gptq_block_kernel<true, 16><<<nb, 16 * LPR, 0, s>>>(W, ldw, d_o, a, w, Rt, ldr, scales, zeros,
                                                          n_groups, group, maxq, perm, E, lde,
                                                          nullptr, codes32, d_i);
  } else {
    if (tall)
      gptq_block_kernel<false, 32><<<nb, 32 * LPR, 0, s>>>(W, ldw, d_o, a, w, Rt, ldr, scales, zeros,
                                                           n_groups, group, maxq, perm, E, lde,
                                                           codes, nullptr, d_i);
    else
      gptq_block_kernel<false, 16><<<nb, 16 * LPR, 0, s>>>(W, ldw, d_o, a, w, Rt, ldr, scales, zeros,
                                                           n_groups, group, maxq, perm, E, lde,
                                                           codes, nullptr, d_i);
  }
  return check_launch("gptq_block");
}

}  // namespace qz
