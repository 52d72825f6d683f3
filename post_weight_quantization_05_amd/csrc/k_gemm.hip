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
// them, so tiles stage straight into LDS without a transpose.  Tiles of 128 x 128 per
// 256-thread workgroup, 4 wavefronts each owning 64 x 64 = 2 x 2 blocks of
// v_mfma_f32_32x32x2_f32.  K advances one slab at a time: the next slab of both operands
// is prefetched into registers while the matrix cores work through the current slab in
// LDS, then written to the single, row-padded LDS buffer between two barriers.  One
// wavefront cannot keep a SIMD's matrix core busy on its own, so co-resident workgroups
// cover each other's barrier and LDS-store phases.  Two slab depths: 64 (70 KB of LDS,
// two workgroups per CU, 128 MFMAs per wavefront per slab) and 32 (36 KB, three
// workgroups per CU, so two wavefronts keep a SIMD at full rate while the third stores;
// one 8-deep step's operands live at a time to fit the registers); the launcher picks
// per shape.  The K index within an 8-wide group is split k = 4 * (lane / 32) + e
// between the two lane halves, identically for A and B, so each lane reads one 16-byte
// vector per operand and feeds four MFMAs.  Interior tiles (whole tile and every slab
// inside the matrices) use unchecked vector loads; edge tiles check every element.
#include "qz_internal.h"

namespace qz {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128;
constexpr int kThreads = 256;

__device__ __forceinline__ float4 load4_checked(const float* __restrict__ base, int64_t row,
                                                int64_t nrows, int64_t ld, int64_t k, int64_t K,
                                                bool vec) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (row >= nrows) return v;
  const float* p = base + row * ld + k;
  if (vec && k + 3 < K) return *reinterpret_cast<const float4*>(p);
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

// KB = slab depth: 32 (three workgroups per CU) or 64 (two per CU).  EPI_SUB, whose
// accumulators are loaded from C up front, is bounded at two workgroups per CU with 32-deep
// slabs (64-deep ones fit only one); its interior tiles address C through wave-uniform
// row pointers, which leaves room for a third.
template <int EPI, bool VEC, int KB>
__global__ __launch_bounds__(kThreads, EPI == EPI_SUB ? (KB == 32 ? 2 : 1) : (KB == 32 ? 3 : 2)) void gemm_nt_kernel(
    const GemmArgs g) {
  constexpr int BK = KB;
  constexpr int LDK = BK + 4;                       // padded LDS row (floats): rows 4 banks apart
  constexpr int PER = (BM * BK / 4) / kThreads;     // float4 chunks per operand per thread
  constexpr int CPR = BK / 4;                       // float4 chunks per row
  constexpr int RSTEP = kThreads / CPR;             // rows between a thread's chunks
  __shared__ __attribute__((aligned(16))) float As[BM * LDK];
  __shared__ __attribute__((aligned(16))) float Bs[BN * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const bool interior = VEC && (m0 + BM <= g.M) && (n0 + BN <= g.N) && (g.K % BK == 0);

  // EPI_SUB's interior tiles: C addressed as a wave-uniform row pointer plus one 32-bit lane
  // offset (4 rows of ldc at most)
  const bool c_rows = interior && g.ldc <= (int64_t{1} << 28);
  f32x16 acc[2][2];
  if constexpr (EPI == EPI_SUB) {
    // C -= A B is computed as C + (-A) B with C loaded into the accumulators before the
    // K loop (its latency overlaps the first slab; the epilogue is a plain store).
    // Accumulator layout: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column
    // l%32 of the 32 x 32 block.
    if (c_rows) {
      // Each register's row pointer is wave-uniform and the lane's offset is the same for
      // all 64 registers, so the loads (and the stores at the end) need no per-register
      // addresses: 219 -> 154 registers, and the launch runs at three wavefronts per SIMD.
      const int lofs = static_cast<int>(4 * (lane >> 5) * g.ldc) + (lane & 31);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float* rowp = g.C + (m0 + wm * 64 + mt * 32 + 8 * (r >> 2) + (r & 3)) * g.ldc +
                                n0 + wn * 64 + nt * 32;
            acc[mt][nt][r] = rowp[lofs];
          }
    } else {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int64_t col = n0 + wn * 64 + nt * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * 64 + mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          acc[mt][nt][r] = (row < g.M && col < g.N) ? g.C[row * g.ldc + col] : 0.f;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // thread's chunks: chunk f = tid + 256 i -> row f / CPR, float4 column f % CPR
  const int crow = tid / CPR, ccol = 4 * (tid % CPR);
  float4 ra[PER], rb[PER];
  const float* __restrict__ Ab = g.A + (m0 + crow) * g.lda + ccol;
  const float* __restrict__ Bb = g.B + (n0 + crow) * g.ldb + ccol;
  const int64_t a_step = RSTEP * g.lda, b_step = RSTEP * g.ldb;

  auto gload = [&](int64_t k0) {
    if (interior) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        ra[i] = *reinterpret_cast<const float4*>(Ab + i * a_step + k0);
        rb[i] = *reinterpret_cast<const float4*>(Bb + i * b_step + k0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        ra[i] = load4_checked(g.A, m0 + crow + RSTEP * i, g.M, g.lda, k0 + ccol, g.K, VEC);
        rb[i] = load4_checked(g.B, n0 + crow + RSTEP * i, g.N, g.ldb, k0 + ccol, g.K, VEC);
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float4 va = ra[i];
      if constexpr (EPI == EPI_SUB) va = make_float4(-va.x, -va.y, -va.z, -va.w);
      *reinterpret_cast<float4*>(&As[(crow + RSTEP * i) * LDK + ccol]) = va;
      *reinterpret_cast<float4*>(&Bs[(crow + RSTEP * i) * LDK + ccol]) = rb[i];
    }
  };

  const int64_t nk = ceil_div(g.K, BK);
  gload(0);
  sstore();
  __syncthreads();

  const int lr = lane & 31, lk = 4 * (lane >> 5);
  for (int64_t kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 8) {
      float4 a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const float4*>(&As[(wm * 64 + t * 32 + lr) * LDK + kk + lk]);
        b[t] = *reinterpret_cast<const float4*>(&Bs[(wn * 64 + t * 32 + lr) * LDK + kk + lk]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mt][e], b[nt][e], acc[mt][nt], 0, 0, 0);
      // at three workgroups per CU, one step's operands live at a time (bounds registers)
      if constexpr (KB == 32) __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 1 < nk) {
      __syncthreads();   // every wave is done with the slab in LDS
      sstore();
      __syncthreads();
    }
  }

  // Epilogue.  32x32 accumulator layout: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the block.
  if constexpr (EPI == EPI_DOTROW) {
    // per row: sum over this tile's columns of acc * A[row][col] in fp64, reduced across
    // the 32 lanes of a half-wave (xor pattern) and then across the two column waves in
    // LDS, both in a fixed order
    __syncthreads();   // the operand buffer becomes the row-sum scratch
    double* red = reinterpret_cast<double*>(As);   // [2][BM]
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm * 64 + mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t row = m0 + rl;
        double v = 0.0;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int64_t col = n0 + wn * 64 + nt * 32 + (lane & 31);
          if (row < g.M && col < g.N)
            v += static_cast<double>(acc[mt][nt][r]) * static_cast<double>(g.A[row * g.lda + col]);
        }
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) v += __shfl_xor(v, off);
        if ((lane & 31) == 0) red[wn * BM + rl] = v;
      }
    }
    __syncthreads();
    if (tid < BM && m0 + tid < g.M)
      g.dpart[(m0 + tid) * tn_n + tn] = red[tid] + red[BM + tid];
    return;
  }
  if (EPI == EPI_SUB && c_rows) {
    const int lofs = static_cast<int>(4 * (lane >> 5) * g.ldc) + (lane & 31);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float* rowp = g.C + (m0 + wm * 64 + mt * 32 + 8 * (r >> 2) + (r & 3)) * g.ldc + n0 +
                        wn * 64 + nt * 32;
          rowp[lofs] = acc[mt][nt][r];
        }
    return;
  }
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
        if (EPI == EPI_STORE || EPI == EPI_SUB) *c = v;   // EPI_SUB: acc started from C
        else if (EPI == EPI_ADD) *c = *c + v;
        else if (EPI == EPI_COLSCALE) *c = v * cv;
        else *c = (g.P[row * g.ldp + col] + g.rho * v) * inv;
      }
    }
  }
}

// Slab depth per launch: 32-deep slabs with three workgroups per CU keep the matrix cores
// busier, but they pay when the tiles do not fill whole rounds of 768 resident
// workgroups (the last round runs part-empty) and, as measured, for long K (12288 and
// 25600 ran slower than with 64-deep slabs); 64-deep slabs with two workgroups per CU
// are used otherwise.  EPI_SUB (the short-K GPTQ update) uses 32 at two workgroups per CU.
inline int slab_depth(int epi, int64_t tiles, int64_t K) {
  if (epi == EPI_SUB) return 32;
  return (tiles % (3 * 256) == 0 && K <= 8192) ? 32 : 64;
}

template <int EPI, int KB>
int launch_kb(const GemmArgs& a, int64_t tiles, bool vec, hipStream_t s) {
  if (vec)
    gemm_nt_kernel<EPI, true, KB><<<static_cast<unsigned>(tiles), kThreads, 0, s>>>(a);
  else
    gemm_nt_kernel<EPI, false, KB><<<static_cast<unsigned>(tiles), kThreads, 0, s>>>(a);
  return check_launch("gemm_nt");
}

template <int EPI>
int launch_epi(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  if (tiles > 0x7fffffff) return fail(QZ_EINVAL, "gemm: too many tiles");
  const bool vec = (a.lda % 4 == 0) && (a.ldb % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(a.A) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(a.B) % 16 == 0);
  if (slab_depth(EPI, tiles, a.K) == 32) return launch_kb<EPI, 32>(a, tiles, vec, s);
  return launch_kb<EPI, 64>(a, tiles, vec, s);
}

}  // namespace

int gemm_tile_cols(int64_t N) { return static_cast<int>(ceil_div(N, int64_t{BN})); }

int launch_gemm_nt(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return QZ_OK;
  switch (epi) {
    case EPI_STORE: return launch_epi<EPI_STORE>(a, s);
    case EPI_SUB: return launch_epi<EPI_SUB>(a, s);
    case EPI_COLSCALE: return launch_epi<EPI_COLSCALE>(a, s);
    case EPI_ADMM1: return launch_epi<EPI_ADMM1>(a, s);
    case EPI_ADD: return launch_epi<EPI_ADD>(a, s);
    case EPI_DOTROW:
      if (a.N != a.K || !a.dpart) return fail(QZ_EINVAL, "gemm: row-dot epilogue needs N == K");
      return launch_epi<EPI_DOTROW>(a, s);
  }
  return fail(QZ_EINVAL, "gemm: bad epilogue");
}

}  // namespace qz
