// GPTQ in-block column loop (GPTQ tutorial, section 3, Algorithm 1, the inner loop):
// for every column j of the block [a, b) in the common order,
//     q_j      = grid value of round-to-nearest(w_j)        (the row's static grid)
//     E[:, j]  = (w_j - q_j) / R_jj
//     w[j:b]  -= E[:, j] R[j, j:b]
// The rows are independent (they share only R), so a workgroup owns 64 rows and runs
// the loop for all of them in lock-step.  Four lanes of a quad share one row; lane q
// of the quad keeps columns q, q+4, q+8, ... of the block in registers, so the row's
// 128-column block never leaves the register file.  At step j the owner lane of the
// column rounds it (IEEE fp32 division, half-to-even), forms E, and a DPP quad
// broadcast hands E to the other three lanes; each lane then updates its remaining
// columns with R[j, :] read from LDS (stored lane-deinterleaved so one quad reads 4
// distinct 16-byte vectors, broadcast across the 16 quads of the wavefront).
// The trailing update of the columns after the block is the separate matrix-core
// GEMM (k_gemm.hip).
#include "qz_internal.h"

namespace qz {

namespace {

constexpr int MAXB = 128;        // largest block
constexpr int ROWS = 64;         // rows per workgroup
constexpr int kThreads = 256;    // 4 lanes per row
constexpr int PER = MAXB / 4;    // columns per lane

__device__ __forceinline__ float quad_bcast(float v, int owner) {
  // DPP quad_perm with all four selectors = owner
  const int ctrl = owner * 0x55;
  int r;
  switch (ctrl) {
    case 0x00: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x00, 0xF, 0xF, false); break;
    case 0x55: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x55, 0xF, 0xF, false); break;
    case 0xAA: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xAA, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xFF, 0xF, 0xF, false); break;
  }
  return __int_as_float(r);
}

// Unclamped code rint(x / s) + z, kept inside the int32 range.
__device__ __forceinline__ float quant_code_noclip(float x, float s, float z) {
  const float u = __builtin_rintf(x / s) + z;
  return fminf(fmaxf(u, -2147483648.0f), 2147483520.0f);
}

// NOCLIP: codes are not clamped to [0, 2^b - 1] (the Babai page's no-clipping regime);
// they stay in registers (one per owned column) and are written as int32 to codes32.
template <bool NOCLIP>
__global__ __launch_bounds__(kThreads) void gptq_block_kernel(
    float* __restrict__ W, int64_t ldw, int64_t d_o, int64_t a, int w,
    const float* __restrict__ Rt, int64_t ldr, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int64_t G, int group, float maxq,
    const int32_t* __restrict__ perm, float* __restrict__ E, int64_t lde,
    uint8_t* __restrict__ codes, int32_t* __restrict__ codes32, int64_t d_i) {
  __shared__ __attribute__((aligned(16))) float Rb[MAXB][4][PER];   // Rb[j][q][i] = R[a+j][a+q+4i]
  __shared__ __attribute__((aligned(8))) float2 sz[ROWS][MAXB];      // (scale, zero) of (row, column)
  __shared__ float rinv[MAXB];
  __shared__ uint8_t cs[ROWS][MAXB];

  const int tid = threadIdx.x;
  const int q = tid & 3;
  const int rl = tid >> 2;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * ROWS;
  const int64_t row = row0 + rl;
  const bool rok = row < d_o;

  // R block (upper part, c >= j) into LDS, deinterleaved by lane.
  for (int e = tid; e < MAXB * MAXB; e += kThreads) {
    const int c = e / MAXB, j = e % MAXB;   // j fastest: contiguous reads of Rt row a+c
    float v = 0.f;
    if (c < w && j < w && c >= j) v = Rt[(a + c) * ldr + a + j];
    Rb[j][c & 3][c >> 2] = v;
  }
  for (int j = tid; j < w; j += kThreads) rinv[j] = 1.0f / Rt[(a + j) * ldr + a + j];
  // each row's grid for each block column (groups are ranges of ORIGINAL columns)
  for (int e = tid; e < ROWS * w; e += kThreads) {
    const int r = e / w, c = e % w;
    float2 v = make_float2(1.f, 0.f);
    if (row0 + r < d_o) {
      const int64_t oc = perm ? perm[a + c] : a + c;
      const int64_t gi = (row0 + r) * G + oc / group;
      v = make_float2(scales[gi], static_cast<float>(zeros[gi]));
    }
    sz[r][c] = v;
  }

  float wr[PER];
  float cr[NOCLIP ? PER : 1];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = q + 4 * i;
    wr[i] = (rok && c < w) ? W[row * ldw + a + c] : 0.f;
  }
  __syncthreads();

#pragma unroll
  for (int j = 0; j < MAXB; ++j) {
    if (j < w) {   // uniform branch: blocks narrower than MAXB skip the tail steps
    const int owner = j & 3;
    const int slot = j >> 2;
    // every lane rounds its own value of slot `slot`; only the owner's is used
    const float x = wr[slot];
    const float2 g = sz[rl][4 * slot + q];
    const float c = NOCLIP ? quant_code_noclip(x, g.x, g.y) : quant_code(x, g.x, g.y, maxq);
    const float qv = g.x * (c - g.y);
    const float err = (x - qv) * rinv[j];
    if (q == owner) {
      wr[slot] = err;
      if constexpr (NOCLIP)
        cr[slot] = c;
      else
        cs[rl][j] = static_cast<uint8_t>(c);
    }
    const float e = quad_bcast(err, owner);
    const float* rrow = &Rb[j][q][0];
#pragma unroll
    for (int i = slot; i < PER; ++i) {
      const int col = q + 4 * i;
      if (col > j) wr[i] -= e * rrow[i];
    }
    }
    // keep each step's LDS reads inside the step (bounds register pressure)
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();

  if (rok) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = q + 4 * i;
      if (c < w) E[row * lde + c] = wr[i];
    }
    if constexpr (NOCLIP) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = q + 4 * i;
        if (c >= w) continue;
        const int64_t oc = perm ? perm[a + c] : a + c;
        codes32[row * d_i + oc] = static_cast<int32_t>(cr[i]);
      }
    } else {
      for (int c = q; c < w; c += 4) {
        const int64_t oc = perm ? perm[a + c] : a + c;
        codes[row * d_i + oc] = cs[rl][c];
      }
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
  const unsigned nb = static_cast<unsigned>(ceil_div(d_o, ROWS));
  if (codes32)
    gptq_block_kernel<true><<<nb, kThreads, 0, s>>>(W, ldw, d_o, a, w, Rt, ldr, scales, zeros,
                                                    n_groups, group, maxq, perm, E, lde, nullptr,
                                                    codes32, d_i);
  else
    gptq_block_kernel<false><<<nb, kThreads, 0, s>>>(W, ldw, d_o, a, w, Rt, ldr, scales, zeros,
                                                     n_groups, group, maxq, perm, E, lde, codes,
                                                     nullptr, d_i);
  return check_launch("gptq_block");
}

}  // namespace qz
