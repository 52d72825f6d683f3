// Calibration Hessian H = X^T X + lambda I (ADMM-Q summary, 1. problem formulation)
// with lambda = damp * mean(diag(X^T X)) (damping: GPTQ tutorial, section 2,
// collinear channels) and the diagonal scaling Sigma = diag(H)^(-1/2) (ADMM-Q
// summary, 2. key components).
//
// X is [n x d] bf16, row-major (tokens are rows), so the contraction index runs
// along the OUTER dimension of both operands.  Each workgroup owns one 128 x 128
// tile of the upper triangle (I <= J; the lower triangle is mirrored afterwards, so
// only n d (d + 1) flops are spent up to tile granularity) and one contiguous token
// range (split-K when the triangle alone cannot fill the chip).  A K-step stages 64
// tokens: every thread loads an 8-token x 8-channel bf16 block with 16-byte loads,
// transposes it in registers (perm-style half-word shuffles) and stores it to LDS as
// channel-major rows of 64 tokens, so that each lane then reads the 8 consecutive
// tokens that v_mfma_f32_32x32x16_bf16 wants per operand with one 16-byte LDS read.
// bf16 x bf16 products are exact in fp32; sums accumulate in fp32 in the MFMA.
//
// Partial tiles of the splits go to the workspace and are summed in a fixed order
// (deterministic), then the finalize kernels add lambda to the diagonal, write
// diag/sigma/lambda and mirror the upper triangle.
#include "qz_internal.h"

namespace qz {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef v4i16 __attribute__((address_space(3)))* lds_v4_ptr;

constexpr int HT = 256;          // output tile edge
constexpr int HBK = 32;          // tokens per pipeline stage
constexpr int LDR = HT + 32;     // LDS row (one token) in bf16: 576 bytes, rows 16 banks apart
constexpr int kThreads = 512;    // 8 wavefronts: 4 (rows) x 2 (columns), 64 x 128 each

struct HArgs {
  const uint16_t* X;
  int64_t n, d;
  int64_t n_tiles;      // upper tiles in the schedule
  const int32_t* tiles; // [n_tiles][2] = (I, J), I <= J, in schedule order
  int64_t S;            // token splits
  int64_t chunk;        // tokens per split (multiple of HBK)
  float* partial;       // [S][n_tiles][HT][HT]
  int vec;              // rows of X start on 16-byte boundaries (d % 8 == 0, X aligned)
};

// 16-byte load of 8 channels of one token row (zero outside the matrix).
__device__ __forceinline__ uint4 load8(const uint16_t* __restrict__ X, int64_t row, int64_t n_end,
                                       int64_t col, int64_t d, bool vec_ok) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row >= n_end || col >= d) return v;
  const uint16_t* p = X + row * d + col;
  if (vec_ok && col + 7 < d) return *reinterpret_cast<const uint4*>(p);
  auto el = [&](int i) -> uint32_t { return (col + i < d) ? static_cast<uint32_t>(p[i]) : 0u; };
  v.x = el(0) | (el(1) << 16);
  v.y = el(2) | (el(3) << 16);
  v.z = el(4) | (el(5) << 16);
  v.w = el(6) | (el(7) << 16);
  return v;
}

// MFMA operand for a 32-channel column block [c0, c0+32) of a token-major LDS tile,
// tokens [kb0, kb0+16): lane l gets channel c0 + l%32 at tokens kb0 + 8*(l/32) + 0..7.
// ds_read_b64_tr_b16 hands lane i of each 16-lane group element i%4 of the chunks
// addressed by lanes i/4 + 4e (e = 0..3); so lane s of the group addresses token row
// k + s/4, channels m + 4*(s%4), and lane i receives channel m + i at tokens k..k+3.
__device__ __forceinline__ bf16x8 operand_tr(const uint16_t* tile, int c0, int kb0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int m = c0 + 16 * (g & 1) + 4 * (s & 3);
  const int k = kb0 + 8 * (g >> 1) + (s >> 2);
  const uint16_t* p0 = tile + k * LDR + m;
  const uint16_t* p1 = p0 + 4 * LDR;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)(p1));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

__global__ __launch_bounds__(kThreads, 1) void gram_bf16_kernel(const HArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][HBK * LDR];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][HBK * LDR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;   // rows 64*wm, columns 128*wn

  // Split-major schedule, gathered per XCD: the hardware deals workgroups round-robin
  // to the 8 XCDs, so logical ids are regrouped to give each XCD a contiguous run of
  // (split, tile) pairs -- concurrently resident tiles then read the same token slab
  // and share it through that XCD's L2.
  int64_t pid = blockIdx.x;
  const int64_t nblk = gridDim.x;
  if ((nblk & 7) == 0) pid = (pid & 7) * (nblk >> 3) + (pid >> 3);
  const int64_t split = pid / g.n_tiles, t = pid % g.n_tiles;
  const int64_t I = g.tiles[2 * t], J = g.tiles[2 * t + 1];
  const bool diag = (I == J);
  const int64_t i0 = I * HT, j0 = J * HT;
  const int64_t k_begin = split * g.chunk;
  int64_t k_end = k_begin + g.chunk;
  if (k_end > g.n) k_end = g.n;
  const bool vec_ok = g.vec != 0;

  // Copy roles: a stage is HBK tokens x 256 channels per panel = 1024 chunks of 16 B;
  // threads take 2 chunks of A and 2 of B (diagonal tiles: B is A and is not copied).
  const uint16_t* __restrict__ X = g.X;
  const int64_t d = g.d;
  const int crow0 = tid >> 5, crow1 = (tid + kThreads) >> 5;   // token rows 0..31
  const int ccol = 8 * (tid & 31);                             // channel 0..248
  uint4 va0, va1, vb0 = make_uint4(0u, 0u, 0u, 0u), vb1 = make_uint4(0u, 0u, 0u, 0u);
#define QZ_GLOAD(k0)                                                         \
  do {                                                                       \
    va0 = load8(X, (k0) + crow0, k_end, i0 + ccol, d, vec_ok);               \
    va1 = load8(X, (k0) + crow1, k_end, i0 + ccol, d, vec_ok);               \
    if (!diag) {                                                             \
      vb0 = load8(X, (k0) + crow0, k_end, j0 + ccol, d, vec_ok);             \
      vb1 = load8(X, (k0) + crow1, k_end, j0 + ccol, d, vec_ok);             \
    }                                                                        \
  } while (0)
#define QZ_SSTORE(buf)                                                       \
  do {                                                                       \
    *reinterpret_cast<uint4*>(&As[buf][crow0 * LDR + ccol]) = va0;           \
    *reinterpret_cast<uint4*>(&As[buf][crow1 * LDR + ccol]) = va1;           \
    if (!diag) {                                                             \
      *reinterpret_cast<uint4*>(&Bs[buf][crow0 * LDR + ccol]) = vb0;         \
      *reinterpret_cast<uint4*>(&Bs[buf][crow1 * LDR + ccol]) = vb1;         \
    }                                                                        \
  } while (0)

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int64_t nk = (k_end > k_begin) ? ceil_div(k_end - k_begin, HBK) : 0;
  if (nk > 0) {
    QZ_GLOAD(k_begin);
    QZ_SSTORE(0);
  }
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = static_cast<int>(kt & 1);
    if (kt + 1 < nk) QZ_GLOAD(k_begin + (kt + 1) * HBK);
    const uint16_t* as = As[buf];
    const uint16_t* bs = diag ? As[buf] : Bs[buf];
#pragma unroll
    for (int ks = 0; ks < HBK; ks += 16) {
      bf16x8 a[2], b[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) a[mt] = operand_tr(as, wm * 64 + mt * 32, ks, lane);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) b[nt] = operand_tr(bs, wn * 128 + nt * 32, ks, lane);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
    }
    if (kt + 1 < nk) QZ_SSTORE(buf ^ 1);
    __syncthreads();
  }
#undef QZ_GLOAD
#undef QZ_SSTORE

  // Partial tile, dense [HT][HT] at (split, tile).  Accumulator layout of a 32x32
  // block: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  float* out = g.partial + (split * g.n_tiles + t) * (static_cast<int64_t>(HT) * HT);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int c = wn * 128 + nt * 32 + (lane & 31);
        out[row * HT + c] = acc[mt][nt][r];
      }
}

// ---------------------------------------------------------------------------------
// Main path (d % 8 == 0): the same tile, but X streams from HBM straight into a
// ring of four 32-token stage buffers with global_load_lds_dwordx4 (lane i of a
// wavefront lands at base + 16 i), so the next 64 tokens stream in while the matrix
// cores work on the current 64.  LDS rows are one token of 256 channels (512 B, no padding);
// the 32-byte chunk c of row r is stored at chunk c ^ (2 (r & 3)), which keeps both
// the transpose reads (4 rows x 2 chunks per half wave) and the DMA writes free of
// bank conflicts.
constexpr int NSTAGE = 4;
constexpr int PANEL = HBK * HT;   // bf16 elements per panel per stage

__device__ __forceinline__ int swz(int k, int m) {   // element offset of (token k, channel m)
  return k * HT + 16 * ((m >> 4) ^ (2 * (k & 3))) + (m & 15);
}

__device__ __forceinline__ bf16x8 operand_swz(const uint16_t* tile, int c0, int kb0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int m = c0 + 16 * (g & 1) + 4 * (s & 3);
  const int k = kb0 + 8 * (g >> 1) + (s >> 2);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)(tile + swz(k, m)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)(tile + swz(k + 4, m)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// One stage of one panel: 32 token rows = 16 row pairs; wavefront w copies pairs w, w+8.
__device__ __forceinline__ void dma_panel(uint16_t* dst, const uint16_t* __restrict__ X,
                                          int64_t k0, int64_t k_end, int64_t col0, int64_t d,
                                          int wave, int lane) {
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int r0 = 2 * (wave + 8 * rep);
    const int r = r0 + (lane >> 5);
    const int q = lane & 31;
    const int c = (q >> 1) ^ (2 * (r & 3));
    const int64_t grow = k0 + r;
    const int64_t gcol = col0 + 16 * c + 8 * (q & 1);
    uint16_t* base = dst + r0 * HT;
    if (grow < k_end && gcol < d) {
      // Issued as inline asm so that the compiler does not treat it as an LDS write it
      // must wait for before every later LDS read: the stages are synchronised by the
      // explicit vmcnt waits below.  The instruction has no register result.
      const uint32_t lds_off = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
          reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint16_t*)base)));
      const uint16_t* src = X + grow * d + gcol;
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                   :
                   : "s"(lds_off), "v"(src)
                   : "memory", "m0");
    } else {
      *reinterpret_cast<uint4*>(base + 8 * lane) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// Pipeline: four stage buffers used as two pairs.  After one barrier the wavefronts
// issue the DMA of the next pair of stages (into the pair consumed before the barrier)
// and then run the matrix cores over the current pair (64 tokens: 32 MFMAs per
// wavefront); the next barrier first waits for that DMA.  One barrier per 64 tokens
// keeps the two wavefronts of a SIMD from stalling in lock-step on every 32 tokens.
__global__ __launch_bounds__(kThreads, 1) void gram_bf16_dma_kernel(const HArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t L0[2 * PANEL];
  __shared__ __attribute__((aligned(16))) uint16_t L1[2 * PANEL];
  __shared__ __attribute__((aligned(16))) uint16_t L2[2 * PANEL];
  __shared__ __attribute__((aligned(16))) uint16_t L3[2 * PANEL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int64_t pid = blockIdx.x;
  const int64_t nblk = gridDim.x;
  if ((nblk & 7) == 0) pid = (pid & 7) * (nblk >> 3) + (pid >> 3);
  const int64_t split = pid / g.n_tiles, t = pid % g.n_tiles;
  const int64_t I = g.tiles[2 * t], J = g.tiles[2 * t + 1];
  const bool diag = (I == J);
  const int64_t i0 = I * HT, j0 = J * HT;
  const int64_t k_begin = split * g.chunk;
  int64_t k_end = k_begin + g.chunk;
  if (k_end > g.n) k_end = g.n;
  const uint16_t* __restrict__ X = g.X;
  const int64_t d = g.d;
  const int64_t nk = (k_end > k_begin) ? ceil_div(k_end - k_begin, HBK) : 0;

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

#define QZ_ISSUE(BUF, kk)                                                                  \
  do {                                                                                     \
    dma_panel(BUF, X, k_begin + (kk) * HBK, k_end, i0, d, wave, lane);                     \
    if (!diag) dma_panel(BUF + PANEL, X, k_begin + (kk) * HBK, k_end, j0, d, wave, lane);  \
  } while (0)

#define QZ_COMPUTE(CUR)                                                                    \
  {                                                                                        \
    const uint16_t* as = CUR;                                                              \
    const uint16_t* bs = diag ? CUR : CUR + PANEL;                                         \
    _Pragma("unroll") for (int ks = 0; ks < HBK; ks += 16) {                               \
      bf16x8 a[2], b[4];                                                                   \
      _Pragma("unroll") for (int mt = 0; mt < 2; ++mt)                                     \
        a[mt] = operand_swz(as, wm * 64 + mt * 32, ks, lane);                              \
      _Pragma("unroll") for (int nt = 0; nt < 4; ++nt)                                     \
        b[nt] = operand_swz(bs, wn * 128 + nt * 32, ks, lane);                             \
      _Pragma("unroll") for (int mt = 0; mt < 2; ++mt)                                     \
        _Pragma("unroll") for (int nt = 0; nt < 4; ++nt)                                   \
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b[nt], acc[mt][nt],  \
                                                                0, 0, 0);                  \
    }                                                                                      \
  }

// vmcnt(0) (the pair's DMA landed) and lgkmcnt(0) (zero fills and this wave's LDS reads
// done), then the workgroup barrier.  s_waitcnt 0x0070: vmcnt 0, expcnt 7, lgkmcnt 0.
#define QZ_PAIR(kk, C0, C1, N0, N1)                                                        \
  if ((kk) < nk) {                                                                         \
    __builtin_amdgcn_s_waitcnt(0x0070);                                                    \
    __builtin_amdgcn_s_barrier();                                                          \
    if ((kk) + 2 < nk) QZ_ISSUE(N0, (kk) + 2);                                             \
    if ((kk) + 3 < nk) QZ_ISSUE(N1, (kk) + 3);                                             \
    QZ_COMPUTE(C0)                                                                         \
    if ((kk) + 1 < nk) QZ_COMPUTE(C1)                                                      \
  }

  if (0 < nk) QZ_ISSUE(L0, 0);
  if (1 < nk) QZ_ISSUE(L1, 1);
  for (int64_t kt = 0; kt < nk; kt += NSTAGE) {
    QZ_PAIR(kt + 0, L0, L1, L2, L3)
    QZ_PAIR(kt + 2, L2, L3, L0, L1)
  }
#undef QZ_PAIR
#undef QZ_COMPUTE
#undef QZ_ISSUE

  float* out = g.partial + (split * g.n_tiles + t) * (static_cast<int64_t>(HT) * HT);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int c = wn * 128 + nt * 32 + (lane & 31);
        out[row * HT + c] = acc[mt][nt][r];
      }
}

// Tile schedule: upper tiles (I <= J) grouped in 8 x 8 super-tiles, so that tiles
// resident at the same time on an XCD share few row and column panels.
__global__ void schedule_kernel(int64_t T, int32_t* __restrict__ tiles) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  constexpr int64_t SB = 8;
  const int64_t nS = ceil_div(T, SB);
  int64_t k = 0;
  for (int64_t SI = 0; SI < nS; ++SI)
    for (int64_t SJ = SI; SJ < nS; ++SJ)
      for (int64_t i = SI * SB; i < (SI + 1) * SB && i < T; ++i)
        for (int64_t j = SJ * SB; j < (SJ + 1) * SB && j < T; ++j)
          if (i <= j) {
            tiles[2 * k] = static_cast<int32_t>(i);
            tiles[2 * k + 1] = static_cast<int32_t>(j);
            ++k;
          }
}

constexpr int kSmall = 256;   // threads of the auxiliary kernels below

// Sum the split partials of every upper tile into H (adding the previous raw sum when
// accumulating), fixed order.  One thread per tile element.
__global__ __launch_bounds__(kSmall) void gram_reduce_kernel(const float* __restrict__ partial,
                                                             int64_t S, int64_t n_tiles,
                                                             const int32_t* __restrict__ tiles,
                                                             int64_t d, int accumulate,
                                                             float* __restrict__ H) {
  const int64_t per_tile = static_cast<int64_t>(HT) * HT;
  const int64_t total = n_tiles * per_tile;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = e / per_tile, rc = e % per_tile;
    const int64_t i = static_cast<int64_t>(tiles[2 * t]) * HT + rc / HT;
    const int64_t j = static_cast<int64_t>(tiles[2 * t + 1]) * HT + rc % HT;
    if (i >= d || j >= d) continue;
    float s = 0.f;
    for (int64_t sp = 0; sp < S; ++sp) s += partial[(sp * n_tiles + t) * per_tile + rc];
    if (accumulate) s += H[i * d + j];
    H[i * d + j] = s;
  }
}

// lambda = damp * mean(diag); H_ii += lambda; diag, sigma.  One workgroup, fp64
// sums in a fixed order.
__global__ __launch_bounds__(kSmall) void lambda_kernel(float* __restrict__ H, int64_t d,
                                                        float damp, float* __restrict__ diag,
                                                        float* __restrict__ sigma,
                                                        float* __restrict__ lambda_out) {
  __shared__ double red[kSmall];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += blockDim.x) s += static_cast<double>(H[i * d + i]);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kSmall / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float lam = static_cast<float>(static_cast<double>(damp) * (red[0] / static_cast<double>(d)));
  for (int64_t i = threadIdx.x; i < d; i += blockDim.x) {
    const float h = H[i * d + i] + lam;
    H[i * d + i] = h;
    if (diag) diag[i] = h;
    if (sigma) sigma[i] = 1.0f / sqrtf(h);
  }
  if (threadIdx.x == 0 && lambda_out) *lambda_out = lam;
}

// H[j][i] = H[i][j] for i < j, through 32 x 32 LDS tiles (coalesced both ways).
__global__ __launch_bounds__(kSmall) void mirror_kernel(float* __restrict__ H, int64_t d) {
  __shared__ float t[32][33];
  const int64_t bi = blockIdx.y, bj = blockIdx.x;   // destination tile (bi, bj), bi >= bj
  if (bj > bi) return;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int64_t i = bj * 32 + r, j = bi * 32 + tx;
    t[r][tx] = (i < d && j < d) ? H[i * d + j] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t i = bi * 32 + r, j = bj * 32 + tx;   // destination (i, j), want i > j
    if (i < d && j < d && i > j) H[i * d + j] = t[tx][r];
  }
}

__global__ __launch_bounds__(kSmall) void transpose_f32_kernel(const float* __restrict__ in,
                                                               int64_t rows, int64_t cols,
                                                               int64_t ldi, float* __restrict__ out,
                                                               int64_t ldo) {
  __shared__ float t[32][33];
  const int64_t r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) {
    const int64_t i = r0 + r, j = c0 + tx;
    t[r][tx] = (i < rows && j < cols) ? in[i * ldi + j] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t j = c0 + r, i = r0 + tx;   // out[j][i] = in[i][j]
    if (i < rows && j < cols) out[j * ldo + i] = t[tx][r];
  }
}

constexpr int64_t kSlots = 256;   // resident workgroups: one per CU

// Token splits: the smallest S whose rounds of kSlots workgroups waste at most 2% more
// than the best S <= 32 (each workgroup's work shrinks as 1/S).
int64_t splits_for(int64_t n, int64_t n_tiles) {
  int64_t smax = n / (8 * HBK);
  if (smax > 32) smax = 32;
  if (smax < 1) smax = 1;
  double best = 1e300;
  for (int64_t S = 1; S <= smax; ++S) {
    const double cost = static_cast<double>(ceil_div(n_tiles * S, kSlots)) / S;
    if (cost < best) best = cost;
  }
  for (int64_t S = 1; S <= smax; ++S) {
    const double cost = static_cast<double>(ceil_div(n_tiles * S, kSlots)) / S;
    if (cost <= best * 1.02) return S;
  }
  return 1;
}

struct HPlan {
  int64_t T, n_tiles, S, chunk;
  size_t tiles_bytes, partial_bytes;
};

HPlan plan_for(int64_t n, int64_t d) {
  HPlan p;
  p.T = ceil_div(d, HT);
  p.n_tiles = p.T * (p.T + 1) / 2;
  p.S = splits_for(n, p.n_tiles);
  p.chunk = round_up(ceil_div(n > 0 ? n : 1, p.S), HBK);
  p.tiles_bytes = align256(static_cast<size_t>(p.n_tiles) * 2 * sizeof(int32_t));
  p.partial_bytes = align256(static_cast<size_t>(p.S) * p.n_tiles * HT * HT * sizeof(float));
  return p;
}

}  // namespace

int launch_transpose_f32(const float* in, int64_t rows, int64_t cols, int64_t ldi, float* out,
                         int64_t ldo, hipStream_t s) {
  if (rows == 0 || cols == 0) return QZ_OK;
  dim3 grid(static_cast<unsigned>(ceil_div(cols, 32)), static_cast<unsigned>(ceil_div(rows, 32)));
  transpose_f32_kernel<<<grid, kSmall, 0, s>>>(in, rows, cols, ldi, out, ldo);
  return check_launch("transpose_f32");
}

size_t hessian_ws_bytes(int64_t n, int64_t d, int xt) {
  if (xt == QZ_F32) return align256(static_cast<size_t>(round_up(d, 4)) * round_up(n, 4) * 4);
  const HPlan p = plan_for(n, d);
  return p.tiles_bytes + p.partial_bytes;
}

int hessian_build(const void* X, int xt, int64_t n, int64_t d, float damp, uint32_t flags,
                  float* H, float* diag, float* sigma, float* lambda_out, void* ws,
                  size_t ws_bytes, hipStream_t s) {
  const bool accumulate = flags & QZ_H_ACCUMULATE;
  if (xt == QZ_BF16) {
    const HPlan p = plan_for(n, d);
    if (p.n_tiles * p.S > 0x7fffffff) return fail(QZ_EINVAL, "hessian: d too large");
    HArgs g;
    g.X = static_cast<const uint16_t*>(X);
    g.n = n;
    g.d = d;
    g.n_tiles = p.n_tiles;
    g.tiles = reinterpret_cast<int32_t*>(ws);
    g.S = p.S;
    g.chunk = p.chunk;
    g.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + p.tiles_bytes);
    g.vec = (d % 8 == 0) && (reinterpret_cast<uintptr_t>(X) % 16 == 0);
    schedule_kernel<<<1, 64, 0, s>>>(p.T, const_cast<int32_t*>(g.tiles));
    QZ_TRY(check_launch("gram_schedule"));
    {
      ScopedTimer tm(K_HESSIAN_GRAM, s);
      if (g.vec)
        gram_bf16_dma_kernel<<<static_cast<unsigned>(p.n_tiles * p.S), kThreads, 0, s>>>(g);
      else
        gram_bf16_kernel<<<static_cast<unsigned>(p.n_tiles * p.S), kThreads, 0, s>>>(g);
      QZ_TRY(check_launch("gram_bf16"));
    }
    ScopedTimer tm(K_HESSIAN_FINISH, s);
    const int64_t total = p.n_tiles * HT * HT;
    const int nb = static_cast<int>(ceil_div(total, kSmall) > 65536 ? 65536 : ceil_div(total, kSmall));
    gram_reduce_kernel<<<nb, kSmall, 0, s>>>(g.partial, p.S, p.n_tiles, g.tiles, d,
                                             accumulate ? 1 : 0, H);
    QZ_TRY(check_launch("gram_reduce"));
  } else {
    // fp32 input: X^T staged K-contiguous, then the fp32 matrix-core GEMM.
    const int64_t ldt = round_up(n, 4);
    float* Xt = static_cast<float*>(ws);
    QZ_TRY(launch_transpose_f32(static_cast<const float*>(X), n, d, d, Xt, ldt, s));
    GemmArgs a{};
    a.M = d; a.N = d; a.K = n;
    a.A = Xt; a.lda = ldt;
    a.B = Xt; a.ldb = ldt;
    a.C = H; a.ldc = d;
    ScopedTimer tm(K_HESSIAN_GRAM, s);
    QZ_TRY(launch_gemm_nt(accumulate ? EPI_ADD : EPI_STORE, a, s));
  }
  if (!(flags & QZ_H_NO_FINALIZE)) {
    ScopedTimer tm(K_HESSIAN_FINISH, s);
    lambda_kernel<<<1, kSmall, 0, s>>>(H, d, damp, diag, sigma, lambda_out);
    QZ_TRY(check_launch("lambda"));
    const int64_t nt = ceil_div(d, 32);
    dim3 grid(static_cast<unsigned>(nt), static_cast<unsigned>(nt));
    mirror_kernel<<<grid, kSmall, 0, s>>>(H, d);
    QZ_TRY(check_launch("mirror"));
  }
  (void)ws_bytes;
  return QZ_OK;
}

}  // namespace qz
