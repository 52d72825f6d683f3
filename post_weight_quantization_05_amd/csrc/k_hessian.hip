// Calibration Hessian H = X^T X + lambda I (ADMM-Q summary, 1. problem formulation)
// with lambda = damp * mean(diag(X^T X)) (damping: GPTQ tutorial, section 2,
// collinear channels) and the diagonal scaling Sigma = diag(H)^(-1/2) (ADMM-Q
// summary, 2. key components).
//
// X is [n x d] bf16, row-major (tokens are rows), so the contraction index runs
// along the OUTER dimension of both operands.  Each workgroup of the main kernel owns
// one 256 x 256 tile of the upper triangle (I <= J; only n d (d + 1) flops are spent up
// to tile granularity) and one contiguous token range (split-K when the triangle alone
// cannot fill the chip).  X streams from HBM into LDS with global_load_lds (no register
// round trip), token-major with a chunk swizzle, and ds_read_b64_tr_b16 hands every lane
// the 8 consecutive tokens of one channel that v_mfma_f32_32x32x16_bf16 wants per
// operand (the transpose happens in the LDS read); the operands of the next 16-token
// step are read while the matrix cores work through the current one.  What bounds the
// kernel is the stream of X into LDS (the copies alone, with no operand reads, take ~90%
// of the kernel's time), so the tile is as large as the fp32 accumulators allow and the
// work is dealt so that concurrently resident tiles share panels in L2.  bf16 x bf16 products are exact in
// fp32; sums accumulate in fp32 in the MFMA.  X whose rows are not 16-byte aligned goes
// through a kernel that stages the same token-major tiles with register loads (element
// loads at the ragged edge) instead of the direct copies.
//
// Epilogue: the split partials are summed in a fixed order (deterministic) in one pass
// that also mirrors each sub-block into the lower triangle through LDS and copies the
// raw diagonal out contiguously; one small kernel then forms lambda from that diagonal
// (the global mean needs every diagonal tile, hence the second launch) and writes
// H_ii + lambda, diag and sigma; H_scaled = Sigma H Sigma is a third pass, only when
// asked for.
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
constexpr int64_t kSlots = 256;  // resident workgroups of the main kernel: one per CU

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
// bank conflicts: element (token k, channel m) of a panel sits at
// k HT + 16 ((m >> 4) ^ (2 (k & 3))) + (m & 15).
constexpr int NSTAGE = 4;
constexpr int PANEL = HBK * HT;   // bf16 elements per panel per stage

// Stage copy: lane l of wavefront w copies, for each of the two row halves (rep), token
// row 2w + l/32 + 16 rep and the 16-byte piece that lands at byte 16 (l mod 32) of that
// LDS row under the chunk swizzle.  The source is a wave-uniform base in scalar
// registers plus one 32-bit lane offset that is the same for every stage and panel.  It is
// issued as inline asm so that the compiler does not treat it as an LDS write it must wait
// for before every later LDS read (the stages are synchronised by the explicit vmcnt waits
// before each barrier); the instruction has no register result.  In
// a stage that lies wholly inside X every lane copies; otherwise lanes whose token row is
// at or past k_end, or whose 8 channels are at or past d, write zeros instead (with
// d % 8 == 0 a 16-byte piece is wholly inside or wholly outside).
__device__ __forceinline__ void dma_row(uint16_t* dst_row, const uint16_t* src, uint32_t voff) {
  const uint32_t lds_off = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint16_t*)dst_row)));
  // The base must sit in scalar registers (the instruction's saddr operand); it is
  // wave-uniform, and readfirstlane makes that explicit to the compiler.
  const uint64_t sa = reinterpret_cast<uint64_t>(src);
  // (readfirstlane returns int: each half goes through uint32_t so that widening the
  // low half cannot sign-extend into the high half.)
  const uint32_t s_lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(sa)));
  const uint32_t s_hi =
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(sa >> 32)));
  const uint64_t su = (static_cast<uint64_t>(s_hi) << 32) | s_lo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_off), "v"(voff), "s"(reinterpret_cast<const uint16_t*>(su))
               : "memory", "m0");
}

// Pipeline: four stage buffers used as two pairs (64 tokens each); operands are
// double-buffered in registers, so the transposing LDS reads for the next 16-token
// step are in flight while the matrix cores work through the current one.  One
// barrier per pair, placed before the pair's last step (whose operands are already in
// registers): once every wavefront has passed it, the pair's buffers are free for the
// copies of the pair after next, and the next pair's copies (waited for just before the
// barrier) are visible, so its first operands are read before the last step's MFMAs;
// the copies of the pair after next are issued behind those MFMAs.
__global__ __launch_bounds__(kThreads, 1) void gram_bf16_dma_kernel(const HArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t Ls[NSTAGE * 2 * PANEL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Work items in split-major order, dealt per round of kSlots resident workgroups: the
  // hardware deals workgroups round-robin to the 8 XCDs, so within each full round the
  // logical ids are regrouped to give every XCD 32 consecutive items (a compact group of
  // tiles, sharing panels through that XCD's L2), while all XCDs stay on the same one or
  // two token splits (sharing them in the last-level cache and in DRAM pages).
  int64_t pid = blockIdx.x;
  const int64_t nblk = gridDim.x;
  {
    const int64_t r = pid / kSlots, in = pid % kSlots;
    if ((r + 1) * kSlots <= nblk) pid = r * kSlots + (in & 7) * (kSlots / 8) + (in >> 3);
  }
  const int64_t split = pid / g.n_tiles, t = pid % g.n_tiles;
  const int64_t I = g.tiles[2 * t], J = g.tiles[2 * t + 1];
  const bool diag = (I == J);
  const int64_t i0 = I * HT, j0 = J * HT;
  const int64_t k_begin = split * g.chunk;
  int64_t k_end = k_begin + g.chunk;
  if (k_end > g.n) k_end = g.n;
  const int64_t d = g.d;
  const int64_t nk = (k_end > k_begin) ? ceil_div(k_end - k_begin, HBK) : 0;
  const int64_t np = (nk + 1) >> 1;   // pairs; a stage past the token range is zero-filled
  const bool cols_in = (i0 + HT <= d) && (j0 + HT <= d);

  // Copy roles (see dma_row).
  const int crow = 2 * wave + (lane >> 5);
  const int cq = lane & 31;
  const int ccol = 16 * ((cq >> 1) ^ (2 * (crow & 3))) + 8 * (cq & 1);
  const uint32_t voff = static_cast<uint32_t>((crow * d + ccol) * sizeof(uint16_t));
  const bool a_col = i0 + ccol < d, b_col = j0 + ccol < d;
  const uint16_t* __restrict__ xa = g.X + k_begin * d + i0;   // token k_begin, channel i0
  const int64_t jdelta = j0 - i0;

  // Operand roles: byte offsets into Ls of the first transposing read of each operand
  // (stage buffer 0, tokens 0..3 of the step); the other reads add immediates.
  uint32_t aoff[2], boffs[4];
  {
    const int gq = lane >> 4, s = lane & 15;
    const int kl = 8 * (gq >> 1) + (s >> 2);
    const int ml = 16 * (gq & 1) + 4 * (s & 3);
    auto sw = [&](int m) {
      return static_cast<uint32_t>(2 * (kl * HT + 16 * ((m >> 4) ^ (2 * (kl & 3))) + (m & 15)));
    };
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) aoff[mt] = sw(wm * 64 + mt * 32 + ml);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      boffs[nt] = sw(wn * 128 + nt * 32 + ml) + (diag ? 0u : 2u * PANEL);
  }
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* const lbase = (lds_char*)(__attribute__((address_space(3))) uint16_t*)Ls;

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  bf16x8 ra0[2], rb0[4], ra1[2], rb1[4];

#define QZ_ISSUE(BUF, st)                                                                  \
  do {                                                                                     \
    const int64_t kr_ = (st) * HBK;   /* first token row of the stage, from k_begin */     \
    uint16_t* dst_ = Ls + (BUF) * 2 * PANEL;                                               \
    const bool full_ = cols_in && k_begin + kr_ + HBK <= k_end;                            \
    _Pragma("unroll") for (int rep = 0; rep < 2; ++rep) {                                  \
      const uint16_t* src_ = xa + (kr_ + 16 * rep) * d;                                    \
      uint16_t* row_ = dst_ + (2 * wave + 16 * rep) * HT;                                  \
      const bool rin_ = k_begin + kr_ + 16 * rep + crow < k_end;                           \
      if (full_ || (rin_ && a_col)) dma_row(row_, src_, voff);                              \
      else *reinterpret_cast<uint4*>(row_ + 8 * lane) = make_uint4(0u, 0u, 0u, 0u);         \
      if (!diag) {                                                                         \
        if (full_ || (rin_ && b_col)) dma_row(row_ + PANEL, src_ + jdelta, voff);           \
        else *reinterpret_cast<uint4*>(row_ + PANEL + 8 * lane) = make_uint4(0u, 0u, 0u, 0u); \
      }                                                                                    \
    }                                                                                      \
  } while (0)

#define QZ_RD(off) __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)(lbase + (off)))
#define QZ_OP(off)                                                                         \
  __builtin_bit_cast(bf16x8, __builtin_shufflevector(QZ_RD(off), QZ_RD((off) + 8 * HT),    \
                                                     0, 1, 2, 3, 4, 5, 6, 7))
#define QZ_LOAD(BUF, ks, RA, RB)                                                           \
  do {                                                                                     \
    constexpr uint32_t c_ = (BUF) * 4 * PANEL + 2 * (ks) * HT;                              \
    _Pragma("unroll") for (int mt = 0; mt < 2; ++mt) RA[mt] = QZ_OP(aoff[mt] + c_);         \
    _Pragma("unroll") for (int nt = 0; nt < 4; ++nt) RB[nt] = QZ_OP(boffs[nt] + c_);        \
  } while (0)

#define QZ_MFMA(RA, RB)                                                                    \
  do {                                                                                     \
    _Pragma("unroll") for (int mt = 0; mt < 2; ++mt)                                       \
      _Pragma("unroll") for (int nt = 0; nt < 4; ++nt)                                     \
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(RA[mt], RB[nt], acc[mt][nt],  \
                                                              0, 0, 0);                    \
  } while (0)

// The scheduling fences keep each step's reads ahead of the previous step's MFMAs (the
// compiler would otherwise sink them and reuse one register set).  Before the barrier:
// vmcnt(0) (the next pair's copies landed) and lgkmcnt(0) (zero fills and this wave's
// LDS reads done); s_waitcnt 0x0070 = vmcnt 0, expcnt 7, lgkmcnt 0.
#define QZ_FENCE __builtin_amdgcn_sched_barrier(0)
#define QZ_PAIR(pp, C0, C1, N0)                                                            \
  if ((pp) < np) {                                                                         \
    QZ_LOAD(C0, 16, ra1, rb1);                                                             \
    QZ_FENCE;                                                                              \
    QZ_MFMA(ra0, rb0);                                                                     \
    QZ_FENCE;                                                                              \
    QZ_LOAD(C1, 0, ra0, rb0);                                                              \
    QZ_FENCE;                                                                              \
    QZ_MFMA(ra1, rb1);                                                                     \
    QZ_FENCE;                                                                              \
    QZ_LOAD(C1, 16, ra1, rb1);                                                             \
    QZ_FENCE;                                                                              \
    QZ_MFMA(ra0, rb0);                                                                     \
    QZ_FENCE;                                                                              \
    __builtin_amdgcn_s_waitcnt(0x0070);                                                    \
    __builtin_amdgcn_s_barrier();                                                          \
    if ((pp) + 1 < np) QZ_LOAD(N0, 0, ra0, rb0);                                           \
    QZ_FENCE;                                                                              \
    QZ_MFMA(ra1, rb1);                                                                     \
    QZ_FENCE;                                                                              \
    if ((pp) + 2 < np) {                                                                   \
      QZ_ISSUE(C0, 2 * ((pp) + 2));                                                        \
      QZ_ISSUE(C1, 2 * ((pp) + 2) + 1);                                                    \
    }                                                                                      \
  }

  if (np > 0) {
    QZ_ISSUE(0, 0);
    QZ_ISSUE(1, 1);
    if (np > 1) {
      QZ_ISSUE(2, 2);
      QZ_ISSUE(3, 3);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
    QZ_LOAD(0, 0, ra0, rb0);
  }
  for (int64_t p = 0; p < np; p += 2) {
    QZ_PAIR(p, 0, 1, 2)
    QZ_PAIR(p + 1, 2, 3, 0)
  }
#undef QZ_PAIR
#undef QZ_FENCE
#undef QZ_MFMA
#undef QZ_LOAD
#undef QZ_OP
#undef QZ_RD
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

// Split-K reduction and mirror in one pass.  One workgroup per 64 x 64 sub-block of an
// upper tile: the S partials of each element are summed in split order (deterministic;
// the previous raw sum is added when accumulating) and written to the upper triangle;
// the sub-block then goes through LDS and is written transposed into the lower triangle
// (both writes coalesced), and diagonal elements are also copied to `dg` (contiguous,
// for the damping kernel).  Sub-blocks below the diagonal of a diagonal tile hold
// nothing the upper triangle does not, and return at once.
constexpr int RSB = 64;   // sub-block edge
__global__ __launch_bounds__(kSmall) void reduce_mirror_kernel(const float* __restrict__ partial,
                                                               int64_t S, int64_t n_tiles,
                                                               const int32_t* __restrict__ tiles,
                                                               int64_t d, int accumulate,
                                                               int mirror, float* __restrict__ H,
                                                               float* __restrict__ dg) {
  __shared__ float tr[RSB][RSB + 1];
  constexpr int per = HT / RSB;
  const int64_t t = blockIdx.x / (per * per);
  const int sb = static_cast<int>(blockIdx.x % (per * per));
  const int sbi = sb / per, sbj = sb % per;
  const int64_t I = tiles[2 * t], J = tiles[2 * t + 1];
  if (I == J && sbi > sbj) return;
  const int64_t r0 = I * HT + sbi * RSB, c0 = J * HT + sbj * RSB;
  if (r0 >= d || c0 >= d) return;
  const int tx = threadIdx.x % RSB, ty = threadIdx.x / RSB;
  constexpr int rstep = kSmall / RSB;
  const int64_t per_tile = static_cast<int64_t>(HT) * HT;
  for (int rr = ty; rr < RSB; rr += rstep) {
    const int64_t i = r0 + rr, j = c0 + tx;
    const int64_t off = static_cast<int64_t>(sbi * RSB + rr) * HT + sbj * RSB + tx;
    float v = 0.f;
    for (int64_t sp = 0; sp < S; ++sp) v += partial[(sp * n_tiles + t) * per_tile + off];
    if (i < d && j < d && i <= j) {
      if (accumulate) v += H[i * d + j];
      H[i * d + j] = v;
      if (i == j) dg[i] = v;
    }
    tr[rr][tx] = v;
  }
  if (!mirror) return;
  __syncthreads();
  for (int rr = ty; rr < RSB; rr += rstep) {
    const int64_t i = c0 + rr, j = r0 + tx;   // destination (i, j) below the diagonal
    if (i < d && j < d && i > j) H[i * d + j] = tr[tx][rr];
  }
}

// lambda = damp * mean(diag), summed in fp64 in a fixed order by one workgroup over the
// raw diagonal (contiguous `dg`, or the diagonal of H when dg is null); then
// H_ii = raw_ii + lambda, diag, sigma = 1 / sqrt(H_ii), lambda_out.
constexpr int kLam = 1024;
__global__ __launch_bounds__(kLam) void lambda_kernel(float* __restrict__ H, int64_t d,
                                                      const float* __restrict__ dg, float damp,
                                                      float* __restrict__ diag,
                                                      float* __restrict__ sigma,
                                                      float* __restrict__ lambda_out,
                                                      float* __restrict__ sig_ws) {
  __shared__ double red[kLam];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += kLam)
    s += static_cast<double>(dg ? dg[i] : H[i * d + i]);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kLam / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float lam = static_cast<float>(static_cast<double>(damp) * (red[0] / static_cast<double>(d)));
  for (int64_t i = threadIdx.x; i < d; i += kLam) {
    const float h = (dg ? dg[i] : H[i * d + i]) + lam;
    const float sg = 1.0f / sqrtf(h);
    H[i * d + i] = h;
    if (diag) diag[i] = h;
    if (sigma) sigma[i] = sg;
    sig_ws[i] = sg;
  }
  if (threadIdx.x == 0 && lambda_out) *lambda_out = lam;
}

// H_scaled = Sigma H Sigma in fp32 from the sigma the damping kernel wrote (Sigma_i =
// 1 / sqrt(H_ii), the rounding of the sigma output), one workgroup per row.
__global__ __launch_bounds__(kSmall) void scaled_kernel(const float* __restrict__ H, int64_t d,
                                                        const float* __restrict__ sg,
                                                        float* __restrict__ Hs) {
  for (int64_t i = blockIdx.x; i < d; i += gridDim.x) {
    const float si = sg[i];
    for (int64_t j = threadIdx.x; j < d; j += kSmall) Hs[i * d + j] = H[i * d + j] * si * sg[j];
  }
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

// Workspace: [X^T staging (fp32 input) | schedule, split partials, raw diagonal (bf16)]
// followed by sigma (d floats) for the H_scaled pass.
size_t hessian_ws_bytes(int64_t n, int64_t d, int xt) {
  const size_t vec = align256(static_cast<size_t>(d) * sizeof(float));
  if (xt == QZ_F32) return align256(static_cast<size_t>(round_up(d, 4)) * round_up(n, 4) * 4) + vec;
  const HPlan p = plan_for(n, d);
  return p.tiles_bytes + p.partial_bytes + 2 * vec;
}

int hessian_build(const void* X, int xt, int64_t n, int64_t d, float damp, uint32_t flags,
                  float* H, float* diag, float* sigma, float* H_scaled, float* lambda_out,
                  void* ws, size_t ws_bytes, hipStream_t s) {
  const bool accumulate = flags & QZ_H_ACCUMULATE;
  const bool finalize = !(flags & QZ_H_NO_FINALIZE);
  const size_t vec = align256(static_cast<size_t>(d) * sizeof(float));
  float* dg = nullptr;   // raw diagonal, contiguous (bf16 path)
  float* sg = reinterpret_cast<float*>(static_cast<char*>(ws) + hessian_ws_bytes(n, d, xt) - vec);
  if (xt == QZ_BF16) {
    const HPlan p = plan_for(n, d);
    if (p.n_tiles * p.S > 0x7fffffff || p.n_tiles * (HT / RSB) * (HT / RSB) > 0x7fffffff)
      return fail(QZ_EINVAL, "hessian: d too large");
    HArgs g;
    g.X = static_cast<const uint16_t*>(X);
    g.n = n;
    g.d = d;
    g.n_tiles = p.n_tiles;
    g.tiles = reinterpret_cast<int32_t*>(ws);
    g.S = p.S;
    g.chunk = p.chunk;
    g.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + p.tiles_bytes);
    dg = reinterpret_cast<float*>(static_cast<char*>(ws) + p.tiles_bytes + p.partial_bytes);
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
    const int64_t per = (HT / RSB) * (HT / RSB);
    reduce_mirror_kernel<<<static_cast<unsigned>(p.n_tiles * per), kSmall, 0, s>>>(
        g.partial, p.S, p.n_tiles, g.tiles, d, accumulate ? 1 : 0, finalize ? 1 : 0, H, dg);
    QZ_TRY(check_launch("gram_reduce_mirror"));
  } else {
    // fp32 input: X^T staged K-contiguous, then the fp32 matrix-core GEMM over the full
    // square; the mirror below makes it exactly symmetric.
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
  if (finalize) {
    ScopedTimer tm(K_HESSIAN_FINISH, s);
    if (!dg) {
      const int64_t nt = ceil_div(d, 32);
      dim3 grid(static_cast<unsigned>(nt), static_cast<unsigned>(nt));
      mirror_kernel<<<grid, kSmall, 0, s>>>(H, d);
      QZ_TRY(check_launch("mirror"));
    }
    lambda_kernel<<<1, kLam, 0, s>>>(H, d, dg, damp, diag, sigma, lambda_out, sg);
    QZ_TRY(check_launch("lambda"));
    if (H_scaled) {
      const int64_t nb = d < 65536 ? d : 65536;
      scaled_kernel<<<static_cast<unsigned>(nb), kSmall, 0, s>>>(H, d, sg, H_scaled);
      QZ_TRY(check_launch("h_scaled"));
    }
  }
  (void)ws_bytes;
  return QZ_OK;
}

}  // namespace qz
