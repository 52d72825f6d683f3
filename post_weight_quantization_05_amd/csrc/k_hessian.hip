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

constexpr int HT = 128;         // output tile edge
constexpr int HBK = 64;         // tokens per K-step
constexpr int LDH = HBK + 8;    // LDS row length in bf16 (144 bytes: staggers banks)
constexpr int kThreads = 256;

struct HArgs {
  const uint16_t* X;
  int64_t n, d;
  int64_t T;        // tiles per edge
  int64_t T_up;     // upper tiles
  int64_t chunk;    // tokens per split (multiple of HBK)
  float* partial;   // [S][T_up][HT][HT]
};

__device__ __forceinline__ void upper_tile(int64_t t, int64_t T, int64_t& I, int64_t& J) {
  // row-by-row enumeration of (I, J), I <= J
  int64_t i = 0, start = 0;
  while (start + (T - i) <= t) {
    start += T - i;
    ++i;
  }
  I = i;
  J = i + (t - start);
}

__device__ __forceinline__ uint4 load8(const uint16_t* __restrict__ X, int64_t row, int64_t n_end,
                                       int64_t col, int64_t d, bool vec_ok) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row >= n_end || col >= d) return v;
  const uint16_t* p = X + row * d + col;
  if (vec_ok && col + 7 < d) return *reinterpret_cast<const uint4*>(p);
  uint16_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = (col + i < d) ? p[i] : uint16_t(0);
  v.x = e[0] | (uint32_t(e[1]) << 16);
  v.y = e[2] | (uint32_t(e[3]) << 16);
  v.z = e[4] | (uint32_t(e[5]) << 16);
  v.w = e[6] | (uint32_t(e[7]) << 16);
  return v;
}

__device__ __forceinline__ uint32_t dw(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// In-register transpose of an 8 x 8 block of 16-bit values: in[e] holds row e
// (8 channels), out[m] holds column m (8 tokens).
__device__ __forceinline__ void transpose8x8(const uint4 in[8], uint4 out[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t x = dw(in[2 * p], q), y = dw(in[2 * p + 1], q);
      lo[p] = (x & 0xffffu) | (y << 16);
      hi[p] = (x >> 16) | (y & 0xffff0000u);
    }
    out[2 * q] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    out[2 * q + 1] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  }
}

__global__ __launch_bounds__(kThreads, 2) void gram_bf16_kernel(const HArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][HT * LDH];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][HT * LDH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int64_t I, J;
  upper_tile(blockIdx.x, g.T, I, J);
  const bool diag = (I == J);
  const int64_t i0 = I * HT, j0 = J * HT;
  const int64_t k_begin = blockIdx.y * g.chunk;
  int64_t k_end = k_begin + g.chunk;
  if (k_end > g.n) k_end = g.n;
  const bool vec_ok = (g.d % 8) == 0;

  // Loader role: threads 0..127 stage the A panel (channels i0..), 128..255 the B
  // panel (channels j0..); on diagonal tiles B is A and the second half idles.
  const bool loadB = tid >= 128;
  const int sub = tid & 127;
  const int kg = sub >> 4;   // token group of 8 (0..7)
  const int mg = sub & 15;   // channel group of 8 (0..15)
  const int64_t col = (loadB ? j0 : i0) + 8 * mg;
  const bool active_loader = !(loadB && diag);

  uint4 v[8];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = active_loader ? load8(g.X, k0 + 8 * kg + e, k_end, col, g.d, vec_ok)
                           : make_uint4(0u, 0u, 0u, 0u);
  };
  auto sstore = [&](int buf) {
    if (!active_loader) return;
    uint4 w[8];
    transpose8x8(v, w);
    uint16_t* dst = loadB ? Bs[buf] : As[buf];
#pragma unroll
    for (int m = 0; m < 8; ++m)
      *reinterpret_cast<uint4*>(&dst[(8 * mg + m) * LDH + 8 * kg]) = w[m];
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int64_t nk = (k_end > k_begin) ? ceil_div(k_end - k_begin, HBK) : 0;
  if (nk > 0) {
    gload(k_begin);
    sstore(0);
  }
  __syncthreads();

  const int lr = lane & 31, lk = 8 * (lane >> 5);
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = static_cast<int>(kt & 1);
    if (kt + 1 < nk) gload(k_begin + (kt + 1) * HBK);
    const uint16_t* as = As[buf];
    const uint16_t* bs = diag ? As[buf] : Bs[buf];
#pragma unroll
    for (int ks = 0; ks < HBK; ks += 16) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const bf16x8*>(&as[(wm * 64 + t * 32 + lr) * LDH + ks + lk]);
        b[t] = *reinterpret_cast<const bf16x8*>(&bs[(wn * 64 + t * 32 + lr) * LDH + ks + lk]);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Partial tile, dense [HT][HT] at (split, tile).  Accumulator layout of a 32x32
  // block: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  float* out = g.partial + (static_cast<int64_t>(blockIdx.y) * g.T_up + blockIdx.x) * (HT * HT);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int c = wn * 64 + nt * 32 + (lane & 31);
        out[row * HT + c] = acc[mt][nt][r];
      }
}

// Sum the split partials of every upper tile into H (adding the previous raw sum
// when accumulating).  One thread per tile element.
__global__ __launch_bounds__(kThreads) void gram_reduce_kernel(const float* __restrict__ partial,
                                                               int64_t S, int64_t T, int64_t T_up,
                                                               int64_t d, int accumulate,
                                                               float* __restrict__ H) {
  const int64_t per_tile = HT * HT;
  const int64_t total = T_up * per_tile;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = e / per_tile, rc = e % per_tile;
    int64_t I, J;
    upper_tile(t, T, I, J);
    const int64_t i = I * HT + rc / HT, j = J * HT + rc % HT;
    if (i >= d || j >= d) continue;
    float s = 0.f;
    for (int64_t sp = 0; sp < S; ++sp) s += partial[(sp * T_up + t) * per_tile + rc];
    if (accumulate) s += H[i * d + j];
    H[i * d + j] = s;
  }
}

// lambda = damp * mean(diag); H_ii += lambda; diag, sigma.  One workgroup, fp64
// sums in a fixed order.
__global__ __launch_bounds__(kThreads) void lambda_kernel(float* __restrict__ H, int64_t d,
                                                          float damp, float* __restrict__ diag,
                                                          float* __restrict__ sigma,
                                                          float* __restrict__ lambda_out) {
  __shared__ double red[kThreads];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += blockDim.x) s += static_cast<double>(H[i * d + i]);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
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
__global__ __launch_bounds__(kThreads) void mirror_kernel(float* __restrict__ H, int64_t d) {
  __shared__ float t[32][33];
  const int64_t bi = blockIdx.y, bj = blockIdx.x;   // destination tile (bi, bj), bi >= bj
  if (bj > bi) return;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  // read source tile (bj, bi) from the upper triangle
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

__global__ __launch_bounds__(kThreads) void transpose_f32_kernel(const float* __restrict__ in,
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

int64_t splits_for(int64_t n, int64_t T_up) {
  const int64_t target = 1024;   // ~2 resident workgroups on each of 256 CUs, twice
  int64_t S = ceil_div(target, T_up);
  const int64_t max_by_n = ceil_div(n, 4 * HBK);
  if (S > max_by_n) S = max_by_n;
  if (S > 64) S = 64;
  if (S < 1) S = 1;
  return S;
}

}  // namespace

int launch_transpose_f32(const float* in, int64_t rows, int64_t cols, int64_t ldi, float* out,
                         int64_t ldo, hipStream_t s) {
  if (rows == 0 || cols == 0) return QZ_OK;
  dim3 grid(static_cast<unsigned>(ceil_div(cols, 32)), static_cast<unsigned>(ceil_div(rows, 32)));
  transpose_f32_kernel<<<grid, kThreads, 0, s>>>(in, rows, cols, ldi, out, ldo);
  return check_launch("transpose_f32");
}

size_t hessian_ws_bytes(int64_t n, int64_t d, int xt) {
  if (xt == QZ_F32) return align256(static_cast<size_t>(round_up(d, 4)) * round_up(n, 4) * 4);
  const int64_t T = ceil_div(d, HT);
  const int64_t T_up = T * (T + 1) / 2;
  const int64_t S = splits_for(n, T_up);
  return align256(static_cast<size_t>(S) * T_up * HT * HT * sizeof(float));
}

int hessian_build(const void* X, int xt, int64_t n, int64_t d, float damp, uint32_t flags,
                  float* H, float* diag, float* sigma, float* lambda_out, void* ws,
                  size_t ws_bytes, hipStream_t s) {
  const bool accumulate = flags & QZ_H_ACCUMULATE;
  if (xt == QZ_BF16) {
    HArgs g;
    g.X = static_cast<const uint16_t*>(X);
    g.n = n;
    g.d = d;
    g.T = ceil_div(d, HT);
    g.T_up = g.T * (g.T + 1) / 2;
    const int64_t S = splits_for(n, g.T_up);
    g.chunk = round_up(ceil_div(n, S), HBK);
    g.partial = static_cast<float*>(ws);
    if (g.T_up > 0x7fffffff) return fail(QZ_EINVAL, "hessian: d too large");
    dim3 grid(static_cast<unsigned>(g.T_up), static_cast<unsigned>(S));
    {
      ScopedTimer tm(K_HESSIAN_GRAM, s);
      gram_bf16_kernel<<<grid, kThreads, 0, s>>>(g);
      QZ_TRY(check_launch("gram_bf16"));
    }
    ScopedTimer tm(K_HESSIAN_FINISH, s);
    const int64_t total = g.T_up * HT * HT;
    int nb = static_cast<int>(ceil_div(total, kThreads) > 65536 ? 65536 : ceil_div(total, kThreads));
    gram_reduce_kernel<<<nb, kThreads, 0, s>>>(g.partial, S, g.T, g.T_up, d, accumulate ? 1 : 0, H);
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
    lambda_kernel<<<1, kThreads, 0, s>>>(H, d, damp, diag, sigma, lambda_out);
    QZ_TRY(check_launch("lambda"));
    const int64_t nt = ceil_div(d, 32);
    dim3 grid(static_cast<unsigned>(nt), static_cast<unsigned>(nt));
    mirror_kernel<<<grid, kThreads, 0, s>>>(H, d);
    QZ_TRY(check_launch("mirror"));
  }
  (void)ws_bytes;
  return QZ_OK;
}

}  // namespace qz
