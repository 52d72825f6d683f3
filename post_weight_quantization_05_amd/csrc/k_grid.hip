// Grid fit, round-to-nearest, code packing and small conversion kernels.
//
// The quantization grid is per (row, group of g consecutive columns), asymmetric,
// b bits (ADMM-Q summary, 1. problem formulation: the set Q; GPTQ tutorial, section
// 3: the grid is an input of Algorithm 1).  The fit reading (range forced to hold 0,
// fp32 arithmetic, half-to-even rounding) is documented in include/qz.h; these
// kernels reproduce it bit for bit.  Everything here is HBM-bound streaming work.
#include "qz_internal.h"

namespace qz {

namespace {

constexpr int kThreads = 256;

inline int blocks_for(int64_t n, int per_block, int cap = 1 << 20) {
  int64_t b = ceil_div(n, per_block);
  if (b < 1) b = 1;
  return static_cast<int>(b > cap ? cap : b);
}

__device__ __forceinline__ void grid_from_range(float lo, float hi, float maxq, float& s,
                                                float& z) {
  if (hi == lo) { lo = -1.0f; hi = 1.0f; }
  s = (hi - lo) / maxq;
  z = fminf(fmaxf(__builtin_rintf(-lo / s), 0.0f), maxq);
}

// One thread per (row, group): for small groups.
template <int WT>
__global__ __launch_bounds__(kThreads) void grid_fit_thread(
    const void* __restrict__ W, int64_t rows, int64_t cols, int group, float maxq,
    float* __restrict__ scales, uint8_t* __restrict__ zeros, float* __restrict__ lo0,
    float* __restrict__ hi0, uint32_t* __restrict__ flag) {
  const int64_t G = cols / group;
  const int64_t total = rows * G;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / G, g = t % G;
    const int64_t base = r * cols + g * group;
    float lo = 0.0f, hi = 0.0f;
    bool bad = false;
    for (int i = 0; i < group; ++i) {
      float v = load_w<WT>(W, base + i);
      bad |= !__builtin_isfinite(v);
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
    if (bad && flag) atomicOr(flag, FLAG_NONFINITE);
    float s, z;
    grid_from_range(lo, hi, maxq, s, z);
    scales[t] = s;
    zeros[t] = static_cast<uint8_t>(z);
    if (lo0) {
      float l = lo, h = hi;
      if (h == l) { l = -1.0f; h = 1.0f; }
      lo0[t] = l;
      hi0[t] = h;
    }
  }
}

// One wavefront (64 lanes) per (row, group): for groups of 64+ columns.
template <int WT>
__global__ __launch_bounds__(kThreads) void grid_fit_wave(
    const void* __restrict__ W, int64_t rows, int64_t cols, int group, float maxq,
    float* __restrict__ scales, uint8_t* __restrict__ zeros, float* __restrict__ lo0,
    float* __restrict__ hi0, uint32_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  const int64_t G = cols / group;
  const int64_t total = rows * G;
  const int64_t wpb = blockDim.x / 64;
  for (int64_t t = blockIdx.x * wpb + threadIdx.x / 64; t < total; t += (int64_t)gridDim.x * wpb) {
    const int64_t r = t / G, g = t % G;
    const int64_t base = r * cols + g * group;
    float lo = 0.0f, hi = 0.0f;
    bool bad = false;
    for (int i = lane; i < group; i += 64) {
      float v = load_w<WT>(W, base + i);
      bad |= !__builtin_isfinite(v);
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
    for (int off = 32; off > 0; off >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, off));
      hi = fmaxf(hi, __shfl_xor(hi, off));
    }
    if (__any(bad) && lane == 0 && flag) atomicOr(flag, FLAG_NONFINITE);
    if (lane == 0) {
      float s, z;
      grid_from_range(lo, hi, maxq, s, z);
      scales[t] = s;
      zeros[t] = static_cast<uint8_t>(z);
      if (lo0) {
        float l = lo, h = hi;
        if (h == l) { l = -1.0f; h = 1.0f; }
        lo0[t] = l;
        hi0[t] = h;
      }
    }
  }
}

// Eight consecutive columns of one row per thread (blockIdx.y strides over rows), so no
// thread divides a flat index; the fast path loads the eight weights with one vector
// load (bf16: 16 bytes; fp32: two 16-byte loads).
constexpr int kPer = 8;

template <int WT>
__device__ __forceinline__ void load_row8(const void* __restrict__ W, int64_t off, int64_t n_left,
                                          bool vec, float (&v)[kPer]) {
  if (vec && n_left >= kPer) {
    if constexpr (WT == QZ_BF16) {
      const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + off);
      const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w4[i] << 16);
        v[2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(W) + off);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) v[i] = (i < n_left) ? load_w<WT>(W, off + i) : 0.f;
}

// vec: every row of W starts on a 16-byte boundary (so each 8-column chunk does too)
template <int WT>
__global__ __launch_bounds__(kThreads) void rtn_kernel(const void* __restrict__ W, int64_t rows,
                                                       int64_t cols, int group, float maxq,
                                                       const float* __restrict__ scales,
                                                       const uint8_t* __restrict__ zeros,
                                                       uint8_t* __restrict__ codes, int vec) {
  const int64_t G = cols / group;
  const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * kPer;
  if (c0 >= cols) return;
  const int64_t n_left = cols - c0;
  const bool one_group = (group % kPer == 0);   // the eight columns share one group
  const bool vstore = vec && n_left >= kPer && (cols % kPer == 0);
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    float v[kPer];
    load_row8<WT>(W, r * cols + c0, n_left, vec != 0, v);
    uint8_t c[kPer];
    if (one_group) {
      const int64_t gi = r * G + c0 / group;
      const float sc = scales[gi], z = static_cast<float>(zeros[gi]);
#pragma unroll
      for (int i = 0; i < kPer; ++i) c[i] = static_cast<uint8_t>(quant_code(v[i], sc, z, maxq));
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int64_t gi = r * G + (c0 + i < cols ? c0 + i : cols - 1) / group;
        c[i] = static_cast<uint8_t>(quant_code(v[i], scales[gi], static_cast<float>(zeros[gi]), maxq));
      }
    }
    uint8_t* dst = codes + r * cols + c0;
    if (vstore) {
      uint2 w;
      __builtin_memcpy(&w, c, sizeof(w));
      *reinterpret_cast<uint2*>(dst) = w;
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (i < n_left) dst[i] = c[i];
    }
  }
}

// One thread per packed 32-bit word.
__global__ __launch_bounds__(kThreads) void pack_kernel(const uint8_t* __restrict__ codes,
                                                        int64_t rows, int64_t cols, int bits,
                                                        int64_t words, uint32_t* __restrict__ out) {
  const int64_t total = rows * words;
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / words, w = t % words;
    const int64_t bit0 = w * 32;
    int64_t i0 = bit0 / bits;
    int64_t i1 = (bit0 + 31) / bits;
    if (i1 > cols - 1) i1 = cols - 1;
    uint32_t acc = 0;
    for (int64_t i = i0; i <= i1; ++i) {
      const uint32_t c = codes[r * cols + i] & mask;
      const int64_t sh = i * bits - bit0;
      acc |= sh >= 0 ? (c << sh) : (c >> (-sh));
    }
    out[t] = acc;
  }
}

// Rows of a multiple of 32 codes, 16-byte aligned: 32 codes fill exactly BITS words of
// the row's bit stream (32 BITS bits), so each thread reads one 32-code unit as two
// 16-byte vectors and writes its BITS words; the shifts are compile-time constants.
// Thread t handles unit t % units of row t / units (total < 2^31, 32-bit indices).
template <int BITS>
__global__ __launch_bounds__(kThreads) void pack32_kernel(const uint8_t* __restrict__ codes,
                                                          uint32_t units, uint32_t total,
                                                          uint32_t* __restrict__ out) {
  constexpr uint32_t mask = (1u << BITS) - 1u;
  for (uint32_t t = blockIdx.x * blockDim.x + threadIdx.x; t < total; t += gridDim.x * blockDim.x) {
    const uint32_t r = t / units, u = t - r * units;
    const uint8_t* src = codes + (static_cast<int64_t>(r) * units + u) * 32;
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    const uint4 b = *reinterpret_cast<const uint4*>(src + 16);
    const uint32_t in[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t w[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t c = (in[i >> 2] >> (8 * (i & 3))) & mask;
      const int pos = i * BITS, wi = pos >> 5, sh = pos & 31;
      w[wi] |= c << sh;
      if (sh + BITS > 32) w[wi + 1] |= c >> (32 - sh);
    }
    uint32_t* dst = out + (static_cast<int64_t>(r) * units + u) * BITS;
#pragma unroll
    for (int k = 0; k < BITS; ++k) dst[k] = w[k];
  }
}

// One thread per code.
__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint32_t* __restrict__ in,
                                                          int64_t rows, int64_t cols, int bits,
                                                          int64_t words, uint8_t* __restrict__ codes) {
  const int64_t total = rows * cols;
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / cols, i = e % cols;
    const int64_t p = i * bits;
    const int64_t w = p >> 5;
    const int off = static_cast<int>(p & 31);
    uint32_t v = in[r * words + w] >> off;
    if (off + bits > 32) v |= in[r * words + w + 1] << (32 - off);
    codes[e] = static_cast<uint8_t>(v & mask);
  }
}

template <int WT>
__global__ __launch_bounds__(kThreads) void to_f32_kernel(const void* __restrict__ W, int64_t rows,
                                                          int64_t cols, const int32_t* __restrict__ perm,
                                                          const float* __restrict__ div,
                                                          float* __restrict__ out, int64_t ldo,
                                                          uint32_t* __restrict__ flag, int vec,
                                                          int vout) {
  const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * kPer;
  bool bad = false;
  if (c0 < cols) {
    const int64_t n_left = cols - c0;
    float dv[kPer];
    if (div) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int64_t j = c0 + i < cols ? c0 + i : cols - 1;
        dv[i] = div[perm ? perm[j] : j];
      }
    }
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
      float v[kPer];
      if (perm) {
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          v[i] = (i < n_left) ? load_w<WT>(W, r * cols + perm[c0 + i]) : 0.f;
      } else {
        load_row8<WT>(W, r * cols + c0, n_left, vec != 0, v);
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (div) v[i] = v[i] / dv[i];
        bad |= (i < n_left) && !__builtin_isfinite(v[i]);
      }
      float* dst = out + r * ldo + c0;
      if (vout && n_left >= kPer) {
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          if (i < n_left) dst[i] = v[i];
      }
    }
  }
  if (flag && __any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, FLAG_NONFINITE);
}

inline dim3 row_grid(int64_t rows, int64_t cols) {
  const int64_t gx = ceil_div(cols, static_cast<int64_t>(kThreads) * kPer);
  const int64_t gy = rows < 65535 ? rows : 65535;
  return dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy > 0 ? gy : 1));
}

__global__ __launch_bounds__(kThreads) void finite_kernel(const float* __restrict__ p, int64_t n,
                                                          uint32_t* __restrict__ flag) {
  bool bad = false;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x)
    bad |= !__builtin_isfinite(p[e]);
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, FLAG_NONFINITE);
}

__global__ __launch_bounds__(kThreads) void perm_count_kernel(const int32_t* __restrict__ perm,
                                                              int64_t d, uint32_t* __restrict__ counts,
                                                              uint32_t* __restrict__ flag) {
  for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < d;
       j += (int64_t)gridDim.x * blockDim.x) {
    const int32_t v = perm[j];
    if (v < 0 || v >= d) {
      atomicOr(flag, FLAG_BADARG);
    } else if (atomicAdd(&counts[v], 1u) != 0u) {
      atomicOr(flag, FLAG_BADARG);   // duplicate
    }
  }
}

__global__ __launch_bounds__(kThreads) void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < n;
       j += (int64_t)gridDim.x * blockDim.x)
    p[j] = 0u;
}

// D = s (C - z) - W_hat per element (the dequantized weights' error), fp32.
template <int WT, typename CT>
__global__ __launch_bounds__(kThreads) void dequant_diff_kernel(
    const CT* __restrict__ codes, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const void* __restrict__ W, int64_t rows, int64_t cols,
    int group, float* __restrict__ out, int64_t ldo, uint32_t* __restrict__ flag) {
  const int64_t total = rows * cols;
  const int64_t G = cols / group;
  bool bad = false;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / cols, j = e % cols;
    const int64_t gi = r * G + j / group;
    const float q = scales[gi] * (static_cast<float>(codes[e]) - static_cast<float>(zeros[gi]));
    const float v = q - load_w<WT>(W, e);
    bad |= !__builtin_isfinite(v);
    out[r * ldo + j] = v;
  }
  if (flag && __any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, FLAG_NONFINITE);
}

// row_f[r] = sum_t dpart[r][t] / 2 in order; total = sum_r row_f[r]: per-thread strided
// sums, then a tree in LDS (fixed order).
__global__ __launch_bounds__(kThreads) void rowsum_half_kernel(const double* __restrict__ dpart,
                                                               int64_t rows, int64_t tcols,
                                                               double* __restrict__ row_f,
                                                               double* __restrict__ total) {
  __shared__ double red[kThreads];
  double acc = 0.0;
  for (int64_t r = threadIdx.x; r < rows; r += kThreads) {
    double v = 0.0;
    for (int64_t t = 0; t < tcols; ++t) v += dpart[r * tcols + t];
    v *= 0.5;
    if (row_f) row_f[r] = v;
    acc += v;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) *total = red[0];
}

}  // namespace

int launch_check_perm(const int32_t* perm, int64_t d, uint32_t* counts, uint32_t* flag,
                      hipStream_t s) {
  const int nb = blocks_for(d, kThreads, 4096);
  zero_u32_kernel<<<nb, kThreads, 0, s>>>(counts, d);
  QZ_TRY(check_launch("check_perm.zero"));
  perm_count_kernel<<<nb, kThreads, 0, s>>>(perm, d, counts, flag);
  return check_launch("check_perm");
}

int launch_grid_fit(const void* W, int wt, int64_t rows, int64_t cols, int group, int bits,
                    float* scales, uint8_t* zeros, float* lo0, float* hi0, uint32_t* flag,
                    hipStream_t s) {
  const float maxq = static_cast<float>((1 << bits) - 1);
  const int64_t n = rows * (cols / group);
  if (n == 0) return QZ_OK;
  if (group >= 64) {
    int nb = blocks_for(n, kThreads / 64);
    if (wt == QZ_BF16)
      grid_fit_wave<QZ_BF16><<<nb, kThreads, 0, s>>>(W, rows, cols, group, maxq, scales, zeros, lo0, hi0, flag);
    else
      grid_fit_wave<QZ_F32><<<nb, kThreads, 0, s>>>(W, rows, cols, group, maxq, scales, zeros, lo0, hi0, flag);
  } else {
    int nb = blocks_for(n, kThreads);
    if (wt == QZ_BF16)
      grid_fit_thread<QZ_BF16><<<nb, kThreads, 0, s>>>(W, rows, cols, group, maxq, scales, zeros, lo0, hi0, flag);
    else
      grid_fit_thread<QZ_F32><<<nb, kThreads, 0, s>>>(W, rows, cols, group, maxq, scales, zeros, lo0, hi0, flag);
  }
  return check_launch("grid_fit");
}

int launch_rtn(const void* W, int wt, int64_t rows, int64_t cols, int group, int bits,
               const float* scales, const uint8_t* zeros, uint8_t* codes, hipStream_t s) {
  const float maxq = static_cast<float>((1 << bits) - 1);
  if (rows * cols == 0) return QZ_OK;
  const int64_t esz = (wt == QZ_BF16) ? 2 : 4;
  // vector loads need every row start on a 16-byte boundary; the 8-byte code stores need
  // 8-byte aligned row starts of `codes`
  const int vec = ((cols * esz) % 16 == 0) && (reinterpret_cast<uintptr_t>(W) % 16 == 0) &&
                  (reinterpret_cast<uintptr_t>(codes) % 8 == 0);
  const dim3 grid = row_grid(rows, cols);
  if (wt == QZ_BF16)
    rtn_kernel<QZ_BF16><<<grid, kThreads, 0, s>>>(W, rows, cols, group, maxq, scales, zeros, codes, vec);
  else
    rtn_kernel<QZ_F32><<<grid, kThreads, 0, s>>>(W, rows, cols, group, maxq, scales, zeros, codes, vec);
  return check_launch("rtn");
}

int launch_pack(const uint8_t* codes, int64_t rows, int64_t cols, int bits, uint32_t* out,
                hipStream_t s) {
  const int64_t words = ceil_div(cols * bits, 32);
  const int64_t n = rows * words;
  if (n == 0) return QZ_OK;
  const int64_t units = cols / 32;
  if (cols % 32 == 0 && reinterpret_cast<uintptr_t>(codes) % 16 == 0 &&
      rows * units < (int64_t{1} << 31) && bits >= 1 && bits <= 8) {
    const uint32_t total = static_cast<uint32_t>(rows * units);
    const unsigned grid = blocks_for(total, kThreads, 65536);
    switch (bits) {
#define QZ_PACK32(B)                                                                           \
  case B:                                                                                      \
    pack32_kernel<B><<<grid, kThreads, 0, s>>>(codes, static_cast<uint32_t>(units), total, out); \
    break;
      QZ_PACK32(1) QZ_PACK32(2) QZ_PACK32(3) QZ_PACK32(4)
      QZ_PACK32(5) QZ_PACK32(6) QZ_PACK32(7) QZ_PACK32(8)
#undef QZ_PACK32
    }
    return check_launch("pack32");
  }
  pack_kernel<<<blocks_for(n, kThreads, 65536), kThreads, 0, s>>>(codes, rows, cols, bits, words, out);
  return check_launch("pack");
}

int launch_unpack(const uint32_t* in, int64_t rows, int64_t cols, int bits, uint8_t* codes,
                  hipStream_t s) {
  const int64_t words = ceil_div(cols * bits, 32);
  const int64_t n = rows * cols;
  if (n == 0) return QZ_OK;
  unpack_kernel<<<blocks_for(n, kThreads, 65536), kThreads, 0, s>>>(in, rows, cols, bits, words, codes);
  return check_launch("unpack");
}

int launch_to_f32(const void* W, int wt, int64_t rows, int64_t cols, const int32_t* perm,
                  const float* div, float* out, int64_t ldo, uint32_t* flag, hipStream_t s) {
  if (rows * cols == 0) return QZ_OK;
  const int64_t esz = (wt == QZ_BF16) ? 2 : 4;
  const int vec = ((cols * esz) % 16 == 0) && (reinterpret_cast<uintptr_t>(W) % 16 == 0);
  const int vout = (ldo % 4 == 0) && (reinterpret_cast<uintptr_t>(out) % 16 == 0);
  const dim3 grid = row_grid(rows, cols);
  if (wt == QZ_BF16)
    to_f32_kernel<QZ_BF16><<<grid, kThreads, 0, s>>>(W, rows, cols, perm, div, out, ldo, flag, vec, vout);
  else
    to_f32_kernel<QZ_F32><<<grid, kThreads, 0, s>>>(W, rows, cols, perm, div, out, ldo, flag, vec, vout);
  return check_launch("to_f32");
}

template <typename CT>
static int dequant_diff_any(const CT* codes, const float* scales, const uint8_t* zeros,
                            const void* W, int wt, int64_t rows, int64_t cols, int group,
                            float* out, int64_t ldo, uint32_t* flag, hipStream_t s) {
  const int64_t n = rows * cols;
  if (n == 0) return QZ_OK;
  const int nb = blocks_for(n, kThreads * 4, 65536);
  if (wt == QZ_BF16)
    dequant_diff_kernel<QZ_BF16, CT><<<nb, kThreads, 0, s>>>(codes, scales, zeros, W, rows, cols,
                                                              group, out, ldo, flag);
  else
    dequant_diff_kernel<QZ_F32, CT><<<nb, kThreads, 0, s>>>(codes, scales, zeros, W, rows, cols,
                                                             group, out, ldo, flag);
  return check_launch("dequant_diff");
}

int launch_dequant_diff(const uint8_t* codes, const float* scales, const uint8_t* zeros,
                        const void* W, int wt, int64_t rows, int64_t cols, int group, float* out,
                        int64_t ldo, uint32_t* flag, hipStream_t s) {
  return dequant_diff_any(codes, scales, zeros, W, wt, rows, cols, group, out, ldo, flag, s);
}

int launch_dequant_diff_i32(const int32_t* codes, const float* scales, const uint8_t* zeros,
                            const void* W, int wt, int64_t rows, int64_t cols, int group,
                            float* out, int64_t ldo, uint32_t* flag, hipStream_t s) {
  return dequant_diff_any(codes, scales, zeros, W, wt, rows, cols, group, out, ldo, flag, s);
}

int launch_rowsum_half(const double* dpart, int64_t rows, int64_t tcols, double* row_f,
                       double* total, hipStream_t s) {
  rowsum_half_kernel<<<1, kThreads, 0, s>>>(dpart, rows, tcols, row_f, total);
  return check_launch("rowsum");
}

int launch_check_finite_f32(const float* p, int64_t n, uint32_t* flag, hipStream_t s) {
  if (n == 0) return QZ_OK;
  finite_kernel<<<blocks_for(n, kThreads * 8, 4096), kThreads, 0, s>>>(p, n, flag);
  return check_launch("check_finite");
}

}  // namespace qz
