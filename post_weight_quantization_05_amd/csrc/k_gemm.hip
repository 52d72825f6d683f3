// fp32 matrix-core GEMM with fused epilogues:  C (epi)= A[M x K] * B[N x K]^T.
//
// Used for the dense contractions of both solvers:
//  * the ADMM-Q W-update (ADMM-Q summary, 2. key components, W-update through the
//    eigendecomposition): T = (P + rho M V) / (Lambda + rho) and W~ = T V^T, and the
//    set-up product P = W~_hat V Lambda;
//  * GPTQ's lazy trailing update W[:, b:] -= E R[a:b, b:] (GPTQ tutorial, section 3,
//    the batched update that turns the column loop into matrix products).
//
// Both operands are read K-contiguous ("NT" form), which is how every caller stores
// them, so tiles stage straight into LDS without a transpose.  Tiles of 128 x 128
// per 256-thread workgroup, 4 wavefronts each owning 64 x 64 = 2 x 2 blocks of
// v_mfma_f32_32x32x2_f32; K advances 32 at a time with double-buffered LDS and
// register prefetch of the next slab.  The K index within an 8-wide slab is split
// as k = 4 * (lane / 32) + e between the two lane halves, identically for A and B,
// so each lane reads one 16-byte vector per operand and feeds four MFMAs.
#include "qz_internal.h"

namespace qz {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDK = BK + 4;  // padded LDS row (floats): shifts rows across banks
constexpr int kThreads = 256;

template <bool VEC>
__device__ __forceinline__ float4 load4(const float* __restrict__ base, int64_t row, int64_t nrows,
                                        int64_t ld, int64_t k, int64_t K) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (row >= nrows) return v;
  const float* p = base + row * ld + k;
  if (VEC && k + 3 < K) return *reinterpret_cast<const float4*>(p);
  if (k + 0 < K) v.x = p[0];
  if (k + 1 < K) v.y = p[1];
  if (k + 2 < K) v.z = p[2];
  if (k + 3 < K) v.w = p[3];
  return v;
}

__device__ __forceinline__ void tile_coords(int64_t pid, int64_t tm_n, int64_t tn_n, int64_t& tm,
                                            int64_t& tn) {
  // Groups of 8 row tiles walk the column tiles together so that the A panels of a
  // group and one B panel at a time stay hot in L2.
  constexpr int64_t GM = 8;
  const int64_t per_group = GM * tn_n;
  const int64_t grp = pid / per_group;
  const int64_t first = grp * GM;
  const int64_t gsz = (tm_n - first) < GM ? (tm_n - first) : GM;
  const int64_t in = pid % per_group;
  tm = first + in % gsz;
  tn = in / gsz;
}

template <int EPI, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void gemm_nt_kernel(const GemmArgs g) {
  __shared__ float As[2][BM * LDK];
  __shared__ float Bs[2][BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t tm_n = ceil_div(g.M, BM), tn_n = ceil_div(g.N, BN);
  // XCD-aware order: the hardware deals workgroups round-robin to the 8 XCDs, so
  // consecutive logical tiles are gathered onto one XCD (and its L2).
  int64_t pid = blockIdx.x;
  const int64_t nblk = gridDim.x;
  if ((nblk & 7) == 0) pid = (pid & 7) * (nblk >> 3) + (pid >> 3);
  int64_t tm, tn;
  tile_coords(pid, tm_n, tn_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  float4 ra[4], rb[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + kThreads * i;
      const int row = f >> 3, c4 = f & 7;
      ra[i] = load4<VEC>(g.A, m0 + row, g.M, g.lda, k0 + 4 * c4, g.K);
      rb[i] = load4<VEC>(g.B, n0 + row, g.N, g.ldb, k0 + 4 * c4, g.K);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + kThreads * i;
      const int row = f >> 3, c4 = f & 7;
      *reinterpret_cast<float4*>(&As[buf][row * LDK + 4 * c4]) = ra[i];
      *reinterpret_cast<float4*>(&Bs[buf][row * LDK + 4 * c4]) = rb[i];
    }
  };

  const int64_t nk = ceil_div(g.K, BK);
  gload(0);
  sstore(0);
  __syncthreads();

  const int lr = lane & 31, lk = 4 * (lane >> 5);
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = static_cast<int>(kt & 1);
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const float* as = As[buf];
    const float* bs = Bs[buf];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 8) {
      float4 a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const float4*>(&as[(wm * 64 + t * 32 + lr) * LDK + kk + lk]);
        b[t] = *reinterpret_cast<const float4*>(&bs[(wn * 64 + t * 32 + lr) * LDK + kk + lk]);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mt].x, b[nt].x, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mt].y, b[nt].y, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mt].z, b[nt].z, acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mt].w, b[nt].w, acc[mt][nt], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the block.
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t col = n0 + wn * 64 + nt * 32 + (lane & 31);
    if (col >= g.N) continue;
    float cv = 0.f, inv = 0.f;
    if (EPI == EPI_COLSCALE) cv = g.colv[col];
    if (EPI == EPI_ADMM1) inv = 1.0f / (g.colv[col] + g.rho);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= g.M) continue;
        const float v = acc[mt][nt][r];
        float* c = g.C + row * g.ldc + col;
        if (EPI == EPI_STORE) *c = v;
        else if (EPI == EPI_SUB) *c = *c - v;
        else if (EPI == EPI_ADD) *c = *c + v;
        else if (EPI == EPI_COLSCALE) *c = v * cv;
        else *c = (g.P[row * g.ldp + col] + g.rho * v) * inv;
      }
    }
  }
}

template <int EPI>
int launch_epi(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  if (tiles > 0x7fffffff) return fail(QZ_EINVAL, "gemm: too many tiles");
  const bool vec = (a.lda % 4 == 0) && (a.ldb % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(a.A) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(a.B) % 16 == 0);
  if (vec)
    gemm_nt_kernel<EPI, true><<<static_cast<unsigned>(tiles), kThreads, 0, s>>>(a);
  else
    gemm_nt_kernel<EPI, false><<<static_cast<unsigned>(tiles), kThreads, 0, s>>>(a);
  return check_launch("gemm_nt");
}

}  // namespace

int launch_gemm_nt(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return QZ_OK;
  switch (epi) {
    case EPI_STORE: return launch_epi<EPI_STORE>(a, s);
    case EPI_SUB: return launch_epi<EPI_SUB>(a, s);
    case EPI_COLSCALE: return launch_epi<EPI_COLSCALE>(a, s);
    case EPI_ADMM1: return launch_epi<EPI_ADMM1>(a, s);
    case EPI_ADD: return launch_epi<EPI_ADD>(a, s);
  }
  return fail(QZ_EINVAL, "gemm: bad epilogue");
}

}  // namespace qz
