// ADMM-Q streaming kernels (ADMM-Q summary, 2. key algorithmic components).
//
// admm_project fuses, per iteration, everything after the W-update into one pass
// over the weights, one wavefront per (row, group):
//   grid refresh   -- scale and zero refit from min/max of the continuous iterate
//                     (W~ Sigma), range forced to hold 0 and, by default, clamped
//                     into the group's initial range [lo_0, hi_0] (a range the clamp
//                     closes to a point keeps the group's current grid);
//   D-update       -- C = clamp(rint((W~ + U) Sigma / s) + z): the projection onto the
//                     grid is round-to-nearest in original coordinates;
//                     D~ = s (C - z) / Sigma;
//   dual update    -- U = (U + W~ - D~) * rho_t / rho_{t+1} (multiplier kept across the
//                     penalty schedule rho_t = rho_0 gamma^t);
//   next input     -- M = D~ - U for the next W-update;
//   residuals      -- sum (W~ - D~)^2 and rho_t^2 sum (D~ - D~_prev)^2, reduced per
//                     workgroup in fp64 into a per-iteration partial slot.
// It reads W~, U (fp32) and the previous codes (u8) and writes U, M (fp32) and the
// codes: 18 bytes per weight, the whole iteration's HBM traffic outside the GEMMs.
#include "qz_internal.h"

// No fused multiply-add contraction in this file: D~ = s (C - z) / Sigma and M = D~ - U
// are rounded exactly as written, so a run resumed from its saved state (codes, grid,
// U) rebuilds M bit for bit.
#pragma clang fp contract(off)

namespace qz {

namespace {

constexpr int kThreads = 256;
// Wavefronts of the projection launch: one per three (row, group) pairs, at most
// 131072 (32768 workgroups: many bytes in flight, a few rows per wavefront to spread
// its start-up), rounded down to a multiple of the number of groups per row so that
// every wavefront keeps one column group and strides over rows.
constexpr int64_t kProjWaves = 131072;
__host__ __device__ inline int64_t proj_waves(int64_t G, int64_t d_o) {
  int64_t target = d_o * G / 3;
  if (target > kProjWaves) target = kProjWaves;
  const int64_t per = target / G;
  return (per > 0 ? per : 1) * G;
}

__global__ __launch_bounds__(kThreads) void project_kernel(const AdmmProj p,
                                                           const float* __restrict__ inv_sigma) {
  __shared__ double red[kThreads / 64][2];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int64_t G = p.d_i / p.group;
  const int64_t total = p.d_o * G;
  const float maxq = static_cast<float>((1 << p.bits) - 1);
  const int64_t wpb = kThreads / 64;
  double acc_p = 0.0, acc_d = 0.0;

  for (int64_t t = blockIdx.x * wpb + wid; t < total; t += static_cast<int64_t>(gridDim.x) * wpb) {
    const int64_t r = t / G, g = t % G;
    const int64_t c0 = g * p.group;
    const float* wt = p.Wt + r * p.ldw + c0;
    float* u = p.U + r * p.d_i + c0;
    float* m = p.M + r * p.ldm + c0;
    uint8_t* cd = p.codes + r * p.d_i + c0;
    const float* sg = p.sigma + c0;
    const float* isg = inv_sigma + c0;

    const float s_old = p.scales[t];
    const float z_old = static_cast<float>(p.zeros[t]);
    float s = s_old, z = z_old;
    if (p.refresh) {
      float lo = 0.f, hi = 0.f;
      for (int i = lane; i < p.group; i += 64) {
        float v = wt[i];
        if (p.refresh == 3) v += u[i];
        v *= sg[i];
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
      }
      for (int off = 32; off > 0; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off));
        hi = fmaxf(hi, __shfl_xor(hi, off));
      }
      if (hi == lo) { lo = -1.f; hi = 1.f; }
      if (p.refresh != 2) {
        lo = fmaxf(lo, p.lo0[t]);
        hi = fminf(hi, p.hi0[t]);
      }
      // a range the clamp closes to a point (hi = lo = 0) defines no grid: keep the
      // current one
      if (hi > lo) {
        s = (hi - lo) / maxq;
        z = fminf(fmaxf(__builtin_rintf(-lo / s), 0.f), maxq);
      }
    }
    const float rs = p.rescale ? p.rho / p.rho_next : 1.0f;
    for (int i = lane; i < p.group; i += 64) {
      const float w = wt[i];
      const float uu = u[i];
      const float zv = (w + uu) * sg[i];
      const float c = quant_code(zv, s, z, maxq);
      const float dt = s * (c - z) * isg[i];
      const float dold = s_old * (static_cast<float>(cd[i]) - z_old) * isg[i];
      const float un = (uu + w - dt) * rs;
      u[i] = un;
      m[i] = dt - un;
      cd[i] = static_cast<uint8_t>(c);
      const float ep = w - dt, ed = dt - dold;
      acc_p += static_cast<double>(ep) * ep;
      acc_d += static_cast<double>(ed) * ed;
    }
    if (p.refresh && lane == 0) {
      p.scales[t] = s;
      p.zeros[t] = static_cast<uint8_t>(z);
    }
  }
  // wavefront then workgroup reduction (fixed order)
  for (int off = 32; off > 0; off >>= 1) {
    acc_p += __shfl_xor(acc_p, off);
    acc_d += __shfl_xor(acc_d, off);
  }
  if (lane == 0) {
    red[wid][0] = acc_p;
    red[wid][1] = acc_d;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double sp = 0.0, sd = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) {
      sp += red[w][0];
      sd += red[w][1];
    }
    const double rho = p.rho;
    p.partial[2 * blockIdx.x] = sp;
    p.partial[2 * blockIdx.x + 1] = rho * rho * sd;
  }
}

// Register-resident variant for groups of exactly 64*EPL columns (64, 128, 256): lane l
// owns EPL consecutive columns of the group and loads them once with vector loads (the
// min/max of the refresh comes from the registers, no second pass over memory).
typedef float vf2 __attribute__((ext_vector_type(2)));
typedef float vf4 __attribute__((ext_vector_type(4)));
template <int EPL>
struct Vec;
template <>
struct Vec<1> { typedef float T; typedef uint8_t C; };
template <>
struct Vec<2> { typedef vf2 T; typedef ushort C; };
template <>
struct Vec<4> { typedef vf4 T; typedef uint32_t C; };

template <int EPL>
__device__ __forceinline__ void vload(const float* p, float (&v)[EPL]) {
  typedef typename Vec<EPL>::T T;
  const T x = *reinterpret_cast<const T*>(p);
  __builtin_memcpy(v, &x, sizeof(T));
}
// The streams the projection writes (U, M, codes) are stored with the nontemporal hint:
// nothing reads them again within the launch, and streaming them past the caches
// measured about 2.5% faster than plain stores for the whole kernel.
template <int EPL>
__device__ __forceinline__ void vstore(float* p, const float (&v)[EPL]) {
  typedef typename Vec<EPL>::T T;
  T x;
  __builtin_memcpy(&x, v, sizeof(T));
  __builtin_nontemporal_store(x, reinterpret_cast<T*>(p));
}
template <int EPL>
__device__ __forceinline__ void cload(const uint8_t* p, uint8_t (&c)[EPL]) {
  typedef typename Vec<EPL>::C C;
  const C x = *reinterpret_cast<const C*>(p);
  __builtin_memcpy(c, &x, sizeof(C));
}
template <int EPL>
__device__ __forceinline__ void cstore(uint8_t* p, const uint8_t (&c)[EPL]) {
  typedef typename Vec<EPL>::C C;
  C x;
  __builtin_memcpy(&x, c, sizeof(C));
  __builtin_nontemporal_store(x, reinterpret_cast<C*>(p));
}

// Min and max over the 64 lanes with DPP moves (VALU latency, no LDS round trips): quad
// swaps, half-row and row mirrors, then the row broadcasts; lane 63 ends with the
// result, which is read back as a uniform value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float v) {
  const int x = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(x, x, CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void minmax_step(float& lo, float& hi) {
  lo = fminf(lo, dpp_move<CTRL, ROW_MASK>(lo));
  hi = fmaxf(hi, dpp_move<CTRL, ROW_MASK>(hi));
}
__device__ __forceinline__ void wave_minmax(float& lo, float& hi) {
  minmax_step<0xB1>(lo, hi);         // quad_perm [1,0,3,2]
  minmax_step<0x4E>(lo, hi);         // quad_perm [2,3,0,1]
  minmax_step<0x141>(lo, hi);        // row_half_mirror
  minmax_step<0x140>(lo, hi);        // row_mirror
  minmax_step<0x142, 0xA>(lo, hi);   // row_bcast:15 into rows 1 and 3
  minmax_step<0x143, 0xC>(lo, hi);   // row_bcast:31 into rows 2 and 3
  lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lo), 63));
  hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hi), 63));
}

// Register-resident variant for groups of exactly 64*EPL columns (64, 128, 256): lane l
// owns EPL consecutive columns of the group and loads them once with vector loads (the
// min/max of the refresh comes from the registers, no second pass over memory).  Each
// wavefront keeps one column group (Sigma loaded once) and strides over the rows.  The
// code is rint(x * (1/s)) with the correctly rounded reciprocal of s: it can differ from
// rint(x / s) only where x / s lies within an ulp of a rounding boundary.  Residual
// terms are summed per lane in fp32 over the wavefront's few rows, then in fp64.
template <int EPL>
__global__ __launch_bounds__(kThreads) void project_reg_kernel(const AdmmProj p,
                                                               const float* __restrict__ inv_sigma) {
  __shared__ double red[kThreads / 64][2];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int64_t G = p.d_i / p.group;
  const int64_t nwaves = proj_waves(G, p.d_o);
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wid;
  const float maxq = static_cast<float>((1 << p.bits) - 1);
  const float rs = p.rescale ? p.rho / p.rho_next : 1.0f;
  float sum_p = 0.f, sum_d = 0.f;
  if (w < nwaves) {
    const int64_t gc = w % G;
    const int64_t rstep = nwaves / G;
    const int64_t cc = gc * p.group + lane * EPL;
    float sg[EPL], isg[EPL];
    vload<EPL>(p.sigma + cc, sg);
    vload<EPL>(inv_sigma + cc, isg);
    for (int64_t r = w / G; r < p.d_o; r += rstep) {
      const int64_t t = r * G + gc;
      float wv[EPL], u[EPL];
      uint8_t cd[EPL];
      vload<EPL>(p.Wt + r * p.ldw + cc, wv);
      vload<EPL>(p.U + r * p.d_i + cc, u);
      cload<EPL>(p.codes + r * p.d_i + cc, cd);
      const float s_old = p.scales[t];
      const float z_old = static_cast<float>(p.zeros[t]);
      float s = s_old, z = z_old;
      if (p.refresh) {
        float lo = 0.f, hi = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float v = wv[e];
          if (p.refresh == 3) v += u[e];
          v *= sg[e];
          lo = fminf(lo, v);
          hi = fmaxf(hi, v);
        }
        wave_minmax(lo, hi);
        if (hi == lo) { lo = -1.f; hi = 1.f; }
        if (p.refresh != 2) {
          lo = fmaxf(lo, p.lo0[t]);
          hi = fminf(hi, p.hi0[t]);
        }
        if (hi > lo) {   // a range closed by the clamp keeps the current grid
          s = (hi - lo) / maxq;
          z = fminf(fmaxf(__builtin_rintf(-lo / s), 0.f), maxq);
        }
      }
      const float rcp = 1.0f / s;
      float un[EPL], mm[EPL];
      uint8_t cn[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float zv = (wv[e] + u[e]) * sg[e];
        const float c = fminf(fmaxf(__builtin_rintf(zv * rcp) + z, 0.f), maxq);
        const float dt = s * (c - z) * isg[e];
        const float dold = s_old * (static_cast<float>(cd[e]) - z_old) * isg[e];
        un[e] = (u[e] + wv[e] - dt) * rs;
        mm[e] = dt - un[e];
        cn[e] = static_cast<uint8_t>(c);
        const float ep = wv[e] - dt, ed = dt - dold;
        sum_p += ep * ep;
        sum_d += ed * ed;
      }
      vstore<EPL>(p.U + r * p.d_i + cc, un);
      vstore<EPL>(p.M + r * p.ldm + cc, mm);
      cstore<EPL>(p.codes + r * p.d_i + cc, cn);
      if (p.refresh && lane == 0) {
        p.scales[t] = s;
        p.zeros[t] = static_cast<uint8_t>(z);
      }
    }
  }
  double acc_p = sum_p, acc_d = sum_d;
  for (int off = 32; off > 0; off >>= 1) {
    acc_p += __shfl_xor(acc_p, off);
    acc_d += __shfl_xor(acc_d, off);
  }
  if (lane == 0) {
    red[wid][0] = acc_p;
    red[wid][1] = acc_d;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double sp = 0.0, sd = 0.0;
    for (int k = 0; k < kThreads / 64; ++k) {
      sp += red[k][0];
      sd += red[k][1];
    }
    const double rho = p.rho;
    p.partial[2 * blockIdx.x] = sp;
    p.partial[2 * blockIdx.x + 1] = rho * rho * sd;
  }
}

// Two groups of 128 columns per wavefront: the lower and upper 32 lanes each own one
// group, four consecutive columns per lane (16-byte loads and stores of W~, U, M and
// 4-byte code accesses, half as many memory instructions per byte as one group per
// wavefront).  The refresh's min/max is a 32-lane reduction (the row reductions, then
// row_bcast:15 into rows 1 and 3: lane 31 ends with the lower group's range and lane 63
// with the upper's).  Arithmetic per element is the same as project_reg_kernel's.
// Wavefronts: the launch keeps the one-group kernel's workgroup count (so the partial
// slots per iteration do not depend on the path); each wavefront keeps one pair of groups
// and strides over rows, about 1.5 rows per wavefront on the 12288-row layers (a third as
// many wavefronts, three rows each, measured 10% slower).
__device__ __forceinline__ void half_wave_minmax(float& lo, float& hi) {
  minmax_step<0xB1>(lo, hi);         // quad_perm [1,0,3,2]
  minmax_step<0x4E>(lo, hi);         // quad_perm [2,3,0,1]
  minmax_step<0x141>(lo, hi);        // row_half_mirror
  minmax_step<0x140>(lo, hi);        // row_mirror
  minmax_step<0x142, 0xA>(lo, hi);   // row_bcast:15 into rows 1 and 3
  const float lo_a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lo), 31));
  const float hi_a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hi), 31));
  const float lo_b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lo), 63));
  const float hi_b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hi), 63));
  const bool upper = (threadIdx.x & 63) >= 32;
  lo = upper ? lo_b : lo_a;
  hi = upper ? hi_b : hi_a;
}

__global__ __launch_bounds__(kThreads) void project_pair_kernel(const AdmmProj p,
                                                                const float* __restrict__ inv_sigma) {
  constexpr int EPL = 4;
  __shared__ double red[kThreads / 64][2];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int64_t G = p.d_i / p.group;
  const int64_t G2 = G / 2;
  const int64_t nw1 = proj_waves(G, p.d_o);
  int64_t per = nw1 / G2;
  if (per < 1) per = 1;
  const int64_t nwaves = per * G2;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wid;
  const float maxq = static_cast<float>((1 << p.bits) - 1);
  const float rs = p.rescale ? p.rho / p.rho_next : 1.0f;
  float sum_p = 0.f, sum_d = 0.f;
  if (w < nwaves) {
    const int64_t gp = w % G2;
    const int64_t gc = 2 * gp + (lane >> 5);
    const int64_t cc = gp * 256 + lane * EPL;
    float sg[EPL], isg[EPL];
    vload<EPL>(p.sigma + cc, sg);
    vload<EPL>(inv_sigma + cc, isg);
    for (int64_t r = w / G2; r < p.d_o; r += per) {
      const int64_t t = r * G + gc;
      float wv[EPL], u[EPL];
      uint8_t cd[EPL];
      vload<EPL>(p.Wt + r * p.ldw + cc, wv);
      vload<EPL>(p.U + r * p.d_i + cc, u);
      cload<EPL>(p.codes + r * p.d_i + cc, cd);
      const float s_old = p.scales[t];
      const float z_old = static_cast<float>(p.zeros[t]);
      float s = s_old, z = z_old;
      if (p.refresh) {
        float lo = 0.f, hi = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float v = wv[e];
          if (p.refresh == 3) v += u[e];
          v *= sg[e];
          lo = fminf(lo, v);
          hi = fmaxf(hi, v);
        }
        half_wave_minmax(lo, hi);
        if (hi == lo) { lo = -1.f; hi = 1.f; }
        if (p.refresh != 2) {
          lo = fmaxf(lo, p.lo0[t]);
          hi = fminf(hi, p.hi0[t]);
        }
        if (hi > lo) {   // a range closed by the clamp keeps the current grid
          s = (hi - lo) / maxq;
          z = fminf(fmaxf(__builtin_rintf(-lo / s), 0.f), maxq);
        }
      }
      const float rcp = 1.0f / s;
      float un[EPL], mm[EPL];
      uint8_t cn[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float zv = (wv[e] + u[e]) * sg[e];
        const float c = fminf(fmaxf(__builtin_rintf(zv * rcp) + z, 0.f), maxq);
        const float dt = s * (c - z) * isg[e];
        const float dold = s_old * (static_cast<float>(cd[e]) - z_old) * isg[e];
        un[e] = (u[e] + wv[e] - dt) * rs;
        mm[e] = dt - un[e];
        cn[e] = static_cast<uint8_t>(c);
        const float ep = wv[e] - dt, ed = dt - dold;
        sum_p += ep * ep;
        sum_d += ed * ed;
      }
      vstore<EPL>(p.U + r * p.d_i + cc, un);
      vstore<EPL>(p.M + r * p.ldm + cc, mm);
      cstore<EPL>(p.codes + r * p.d_i + cc, cn);
      if (p.refresh && (lane & 31) == 0) {
        p.scales[t] = s;
        p.zeros[t] = static_cast<uint8_t>(z);
      }
    }
  }
  double acc_p = sum_p, acc_d = sum_d;
  for (int off = 32; off > 0; off >>= 1) {
    acc_p += __shfl_xor(acc_p, off);
    acc_d += __shfl_xor(acc_d, off);
  }
  if (lane == 0) {
    red[wid][0] = acc_p;
    red[wid][1] = acc_d;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double sp = 0.0, sd = 0.0;
    for (int k = 0; k < kThreads / 64; ++k) {
      sp += red[k][0];
      sd += red[k][1];
    }
    const double rho = p.rho;
    p.partial[2 * blockIdx.x] = sp;
    p.partial[2 * blockIdx.x + 1] = rho * rho * sd;
  }
}

// M = s (C - z) / Sigma - U  (U may be null: zero)
__global__ __launch_bounds__(kThreads) void init_m_kernel(const uint8_t* __restrict__ codes,
                                                          const float* __restrict__ scales,
                                                          const uint8_t* __restrict__ zeros,
                                                          const float* __restrict__ U,
                                                          const float* __restrict__ inv_sigma,
                                                          int64_t d_o, int64_t d_i, int group,
                                                          float* __restrict__ M, int64_t ldm) {
  const int64_t G = d_i / group;
  const int64_t total = d_o * d_i;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / d_i, j = e % d_i;
    const int64_t gi = r * G + j / group;
    const float dt = scales[gi] * (static_cast<float>(codes[e]) - static_cast<float>(zeros[gi])) *
                     inv_sigma[j];
    M[r * ldm + j] = dt - (U ? U[e] : 0.f);
  }
}

// One workgroup per iteration: the per-block partial sums are added in a fixed order
// (strided per thread, then a tree in LDS), so the result does not depend on timing.
__global__ __launch_bounds__(kThreads) void residual_kernel(const double* __restrict__ partial,
                                                            int iters, int nblocks,
                                                            float* __restrict__ residuals,
                                                            uint32_t* __restrict__ flag) {
  __shared__ double sp_s[kThreads], sd_s[kThreads];
  const int t = blockIdx.x;
  if (t >= iters) return;
  const double2* q = reinterpret_cast<const double2*>(partial + static_cast<int64_t>(t) * nblocks * 2);
  double sp = 0.0, sd = 0.0;
  for (int b = threadIdx.x; b < nblocks; b += kThreads) {
    const double2 v = q[b];
    sp += v.x;
    sd += v.y;
  }
  sp_s[threadIdx.x] = sp;
  sd_s[threadIdx.x] = sd;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) {
      sp_s[threadIdx.x] += sp_s[threadIdx.x + h];
      sd_s[threadIdx.x] += sd_s[threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float rp = static_cast<float>(sqrt(sp_s[0])), rd = static_cast<float>(sqrt(sd_s[0]));
    if (residuals) {
      residuals[2 * t] = rp;
      residuals[2 * t + 1] = rd;
    }
    if (!__builtin_isfinite(rp) || !__builtin_isfinite(rd)) atomicOr(flag, FLAG_NONFINITE);
  }
}

__global__ __launch_bounds__(kThreads) void fill_kernel(float* __restrict__ p, int64_t n, float v) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x)
    p[e] = v;
}

__global__ __launch_bounds__(kThreads) void inv_kernel(const float* __restrict__ x, int64_t n,
                                                       float* __restrict__ y) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x)
    y[e] = 1.0f / x[e];
}

// lo_0 = s (0 - z), hi_0 = s (2^b - 1 - z) for a caller-supplied grid.
__global__ __launch_bounds__(kThreads) void range_of_grid_kernel(const float* __restrict__ scales,
                                                                 const uint8_t* __restrict__ zeros,
                                                                 int64_t n, float maxq,
                                                                 float* __restrict__ lo0,
                                                                 float* __restrict__ hi0) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const float s = scales[e], z = static_cast<float>(zeros[e]);
    lo0[e] = -s * z;
    hi0[e] = s * (maxq - z);
  }
}

__global__ __launch_bounds__(kThreads) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n,
                                                            uint32_t v) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x)
    p[e] = v;
}

__global__ __launch_bounds__(kThreads) void copy_bytes_kernel(const uint8_t* __restrict__ src,
                                                              int64_t n, uint8_t* __restrict__ dst) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x)
    dst[e] = src[e];
}

inline unsigned grid_for(int64_t n) {
  int64_t b = ceil_div(n, kThreads * 4);
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return static_cast<unsigned>(b);
}

}  // namespace

int admm_proj_blocks(int64_t G, int64_t d_o) {
  return static_cast<int>(ceil_div(proj_waves(G > 0 ? G : 1, d_o > 0 ? d_o : 1), int64_t{kThreads / 64}));
}

int launch_admm_project(const AdmmProj& p, hipStream_t s, const float* inv_sigma) {
  // register-resident path when a group is exactly 64, 128 or 256 columns and every row
  // start is aligned for the vector loads (U, codes and sigma may be the caller's buffers)
  const bool al = (p.d_i % 4 == 0) && (p.ldw % 4 == 0) && (p.ldm % 4 == 0) &&
                  (reinterpret_cast<uintptr_t>(p.U) % 16 == 0) &&
                  (reinterpret_cast<uintptr_t>(p.codes) % 4 == 0) &&
                  (reinterpret_cast<uintptr_t>(p.sigma) % 16 == 0);
  const int nb = admm_proj_blocks(p.d_i / p.group, p.d_o);
  if (al && p.group == 128 && (p.d_i / p.group) % 2 == 0)
    project_pair_kernel<<<nb, kThreads, 0, s>>>(p, inv_sigma);
  else if (al && p.group == 128)
    project_reg_kernel<2><<<nb, kThreads, 0, s>>>(p, inv_sigma);
  else if (al && p.group == 256)
    project_reg_kernel<4><<<nb, kThreads, 0, s>>>(p, inv_sigma);
  else if (p.group == 64)
    project_reg_kernel<1><<<nb, kThreads, 0, s>>>(p, inv_sigma);
  else
    project_kernel<<<nb, kThreads, 0, s>>>(p, inv_sigma);
  return check_launch("admm_project");
}

int launch_admm_init_m(const uint8_t* codes, const float* scales, const uint8_t* zeros,
                       const float* U, const float* inv_sigma, int64_t d_o, int64_t d_i, int group,
                       float* M, int64_t ldm, hipStream_t s) {
  if (d_o * d_i == 0) return QZ_OK;
  init_m_kernel<<<grid_for(d_o * d_i), kThreads, 0, s>>>(codes, scales, zeros, U, inv_sigma, d_o,
                                                          d_i, group, M, ldm);
  return check_launch("admm_init_m");
}

int launch_admm_residuals(const double* partial, int iters, int nblocks, float* residuals,
                          uint32_t* flag, hipStream_t s) {
  if (iters <= 0) return QZ_OK;
  residual_kernel<<<static_cast<unsigned>(iters), kThreads, 0, s>>>(
      partial, iters, nblocks, residuals, flag);
  return check_launch("admm_residuals");
}

int launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n == 0) return QZ_OK;
  fill_kernel<<<grid_for(n), kThreads, 0, s>>>(p, n, v);
  return check_launch("fill_f32");
}

int launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n == 0) return QZ_OK;
  fill_u32_kernel<<<grid_for(n), kThreads, 0, s>>>(p, n, v);
  return check_launch("fill_u32");
}

int launch_inverse_f32(const float* x, int64_t n, float* y, hipStream_t s) {
  if (n == 0) return QZ_OK;
  inv_kernel<<<grid_for(n), kThreads, 0, s>>>(x, n, y);
  return check_launch("inverse_f32");
}

int launch_range_of_grid(const float* scales, const uint8_t* zeros, int64_t n, int bits,
                         float* lo0, float* hi0, hipStream_t s) {
  if (n == 0) return QZ_OK;
  range_of_grid_kernel<<<grid_for(n), kThreads, 0, s>>>(scales, zeros, n,
                                                         static_cast<float>((1 << bits) - 1), lo0, hi0);
  return check_launch("range_of_grid");
}

int launch_copy_bytes(const void* src, int64_t n, void* dst, hipStream_t s) {
  if (n == 0) return QZ_OK;
  copy_bytes_kernel<<<grid_for(n), kThreads, 0, s>>>(static_cast<const uint8_t*>(src), n,
                                                      static_cast<uint8_t*>(dst));
  return check_launch("copy_bytes");
}

}  // namespace qz
