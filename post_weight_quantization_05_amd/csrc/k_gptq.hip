// GPTQ in-block column kernel (GPTQ tutorial, section 3: the column-by-column part of
// the blocked quantizer; section 2 gives the compensation it applies).  Inside a block
// of at most 128 columns the columns are fixed one after another in the common order:
// every row rounds its current value of the column on its static grid, and the error
// divided by the pivot R_jj (kept per row as the block's E) is passed on to the block's
// remaining columns along row j of R.  Columns after the block receive all of the
// block's errors at once, through the separate matrix-core product in k_gemm.hip.
//
// The rows are independent (they share only R), so a workgroup owns 64 rows and steps
// through the columns for all of them together.  Four lanes of a quad share one row;
// lane q of the quad keeps columns q, q+4, q+8, ... of the block in registers, so the
// row's block never leaves the register file.  At step j the lane holding column j
// rounds it (IEEE fp32 division, half-to-even) and forms the scaled error, a DPP quad
// broadcast hands it to the other three lanes, and each lane updates its columns with
// R's row j read from LDS (stored lane-deinterleaved and padded, so the four distinct
// slices a wavefront reads per instruction, and the staging writes, are free of bank
// conflicts).  The workgroup's set-up stages R's block and each row's (scale, zero) per
// column with many global loads in flight (clamped addresses, selected afterwards); at
// the end E leaves through LDS as whole rows and, in natural order, the codes as
// 16-byte row pieces.
#include "qz_internal.h"

namespace qz {

namespace {

constexpr int MAXB = 128;        // largest block
constexpr int ROWS = 64;         // rows per workgroup
constexpr int kThreads = 256;    // 4 lanes per row
constexpr int PER = MAXB / 4;    // columns per lane
constexpr int RQ = PER + 1;      // LDS stride of the four lane slices of an R row
constexpr int RJ = 4 * RQ + 1;   // LDS stride of an R row

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
  // R[a+j][a+q+4i] at Rb[j * RJ + q * RQ + i]: q stride 33 and j stride 133 (5 mod 64
  // banks), so the staging writes (consecutive j across lanes) and the step reads (four
  // q per instruction) are free of bank conflicts
  __shared__ __attribute__((aligned(16))) float Rb[MAXB * RJ];
  __shared__ __attribute__((aligned(16))) float2 sz[ROWS][MAXB];     // (scale, zero) of (row, column)
  __shared__ float rinv[MAXB];
  __shared__ __attribute__((aligned(16))) uint8_t cs[ROWS][MAXB];

  const int tid = threadIdx.x;
  const int q = tid & 3;
  const int rl = tid >> 2;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * ROWS;
  const int64_t row = row0 + rl;
  const bool rok = row < d_o;

  // R block (upper part, c >= j) into LDS, deinterleaved by lane.  Loads are issued 16 at
  // a time from clamped (always valid) addresses and selected afterwards, so their
  // latencies overlap.
  {
    constexpr int RIT = MAXB * MAXB / kThreads;
    constexpr int RU = 16;
#pragma unroll
    for (int it0 = 0; it0 < RIT; it0 += RU) {
      float v[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int e = tid + (it0 + u) * kThreads;
        const int c = e / MAXB, j = e % MAXB;   // j fastest: contiguous reads of Rt row a+c
        const int cc = c < w ? c : w - 1, jj = j < w ? j : w - 1;
        const float x = Rt[(a + cc) * ldr + a + jj];
        v[u] = (c < w && j < w && c >= j) ? x : 0.f;
      }
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int e = tid + (it0 + u) * kThreads;
        const int c = e / MAXB, j = e % MAXB;
        Rb[j * RJ + (c & 3) * RQ + (c >> 2)] = v[u];
      }
    }
  }
  for (int j = tid; j < w; j += kThreads) rinv[j] = 1.0f / Rt[(a + j) * ldr + a + j];
  // each row's grid for each block column (groups are ranges of ORIGINAL columns), 8
  // (row, column) pairs per thread at a time from clamped addresses
  {
    constexpr int GIT = ROWS * MAXB / kThreads;
    constexpr int GU = 16;
    const int64_t last_row = d_o - 1;
#pragma unroll
    for (int it0 = 0; it0 < GIT; it0 += GU) {
      float sv[GU], zv[GU];
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        const int e = tid + (it0 + u) * kThreads;
        const int r = e / MAXB, c = e % MAXB;
        const int cc = c < w ? c : w - 1;
        const int64_t rr = (row0 + r) < last_row ? (row0 + r) : last_row;
        const int64_t oc = perm ? perm[a + cc] : a + cc;
        const int64_t gi = rr * G + oc / group;
        sv[u] = scales[gi];
        zv[u] = static_cast<float>(zeros[gi]);
      }
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        const int e = tid + (it0 + u) * kThreads;
        const int r = e / MAXB, c = e % MAXB;
        sz[r][c] = (row0 + r < d_o) ? make_float2(sv[u], zv[u]) : make_float2(1.f, 0.f);
      }
    }
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
    const float* rrow = &Rb[j * RJ + q * RQ];
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

  // E goes out through LDS (the grid's area is free after the loop) so that each
  // wavefront writes whole rows; rows of Es are 132 floats apart (conflict-free writes)
  {
    constexpr int ES = MAXB + 4;
    float* Es = reinterpret_cast<float*>(&sz[0][0]);
#pragma unroll
    for (int i = 0; i < PER; ++i) Es[rl * ES + q + 4 * i] = wr[i];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (ROWS * MAXB / 4) / kThreads; ++u) {
      const int k = tid + u * kThreads;
      const int r = k / (MAXB / 4), c4 = 4 * (k % (MAXB / 4));
      const int64_t grow = row0 + r;
      if (grow >= d_o || c4 >= w) continue;
      const float4 v = *reinterpret_cast<const float4*>(&Es[r * ES + c4]);
      float* dst = E + grow * lde + c4;
      if (c4 + 3 < w) {
        *reinterpret_cast<float4*>(dst) = v;
      } else {
        dst[0] = v.x;
        if (c4 + 1 < w) dst[1] = v.y;
        if (c4 + 2 < w) dst[2] = v.z;
      }
    }
  }
  if constexpr (NOCLIP) {
    if (rok) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = q + 4 * i;
        if (c >= w) continue;
        const int64_t oc = perm ? perm[a + c] : a + c;
        codes32[row * d_i + oc] = static_cast<int32_t>(cr[i]);
      }
    }
  } else if (!perm && w == MAXB && (d_i % 16) == 0 &&
             (reinterpret_cast<uintptr_t>(codes) & 15) == 0) {
    // natural order, full block: each row's 128 codes are contiguous, 16 bytes per store
#pragma unroll
    for (int u = 0; u < (ROWS * MAXB / 16) / kThreads; ++u) {
      const int k = tid + u * kThreads;
      const int r = k / (MAXB / 16), c16 = 16 * (k % (MAXB / 16));
      const int64_t grow = row0 + r;
      if (grow >= d_o) continue;
      *reinterpret_cast<uint4*>(codes + grow * d_i + a + c16) =
          *reinterpret_cast<const uint4*>(&cs[r][c16]);
    }
  } else if (rok) {
    for (int c = q; c < w; c += 4) {
      const int64_t oc = perm ? perm[a + c] : a + c;
      codes[row * d_i + oc] = cs[rl][c];
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
