// C ABI of libqz (declared and documented in include/qz.h): argument checks,
// workspace layout and the launch sequence of each solver.  Nothing here computes;
// every step runs in the kernels of the k_*.hip translation units.
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>

#include "qz_internal.h"

namespace qz {

namespace {
thread_local std::string g_err;

int read_flag(const uint32_t* flag, hipStream_t s, uint32_t* host) {
  *host = 0;
  QZ_HIP(hipMemcpyAsync(host, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  QZ_HIP(hipStreamSynchronize(s));
  return QZ_OK;
}

bool valid_dtype(int t) { return t == QZ_BF16 || t == QZ_F32; }

int check_grid(const qz_grid* g, int64_t d_i) {
  if (!g) return fail(QZ_EINVAL, "grid is null");
  if (g->struct_size < sizeof(qz_grid)) return fail(QZ_EINVAL, "grid.struct_size too small");
  if (g->bits < 2 || g->bits > 8) return fail(QZ_EINVAL, "grid.bits must be in 2..8");
  if (g->group_size < 1) return fail(QZ_EINVAL, "grid.group_size must be >= 1");
  if (d_i % g->group_size != 0) return fail(QZ_EINVAL, "grid.group_size must divide d_i");
  if (g->flags & ~QZ_GRID_CALLER) return fail(QZ_EINVAL, "grid.flags has unknown bits");
  return QZ_OK;
}

// RTN with the status word at `flag` (device memory, one 32-bit word).
int rtn_run(const void* W, int32_t wt, int64_t d_o, int64_t d_i, const qz_grid* grid,
            uint8_t* codes, float* scales, uint8_t* zeros, uint32_t* flag, hipStream_t stream) {
  QZ_TRY(launch_fill_u32(flag, 1, 0u, stream));
  {
    ScopedTimer tm(K_GRID_RTN, stream);
    if (!(grid->flags & QZ_GRID_CALLER)) {
      QZ_TRY(launch_grid_fit(W, wt, d_o, d_i, grid->group_size, grid->bits, scales, zeros, nullptr,
                             nullptr, flag, stream));
    }
    QZ_TRY(launch_rtn(W, wt, d_o, d_i, grid->group_size, grid->bits, scales, zeros, codes, stream));
  }
  uint32_t h = 0;
  QZ_TRY(read_flag(flag, stream, &h));
  if (h & FLAG_NONFINITE) return fail(QZ_ENONFINITE, "rtn: non-finite weight");
  return QZ_OK;
}

// Scratch of the allocation-free entry point (qz_rtn_noalloc): a file-scope device
// array, one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol); it uses
// the device address that hipGetSymbolAddress returns, looked up once per device with
// that device current and kept.
constexpr size_t kNoAllocScratchBytes = 256;
__device__ __align__(256) uint32_t scratch[kNoAllocScratchBytes / sizeof(uint32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch[kMaxDevices] = {};

int noalloc_scratch(uint32_t** out) {
  int dev = 0;
  QZ_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(QZ_EHIP, "device index out of range");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(QZ_EHIP, std::string("no-alloc scratch: hipGetSymbolAddress failed: ") +
                               hipGetErrorString(e));
    g_scratch[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch[dev];
  return QZ_OK;
}

size_t rtn_ws() {
  Carver c(nullptr);
  c.take<uint32_t>(1);   // status word
  return c.used;
}

size_t objective_ws(int64_t d_o, int64_t d_i) {
  Carver c(nullptr);
  c.take<uint32_t>(1);
  c.take<float>(static_cast<size_t>(d_o) * round_up(d_i, 4));          // D = Q - W_hat
  c.take<double>(static_cast<size_t>(d_o) * gemm_tile_cols(d_i));      // row partials
  c.take<double>(1);                                                    // total
  return c.used;
}

size_t lsearch_ws(int64_t d_o, int64_t d_i, int64_t group) {
  const int64_t G = d_i / group;
  Carver c(nullptr);
  c.take<uint32_t>(1);
  c.take<float>(static_cast<size_t>(d_o) * round_up(d_i, 4));   // D = Q - W_hat
  c.take<float>(static_cast<size_t>(d_o) * round_up(d_i, 4));   // gradient D H
  c.take<float>(static_cast<size_t>(d_o) * G);                   // proposal change
  c.take<int32_t>(static_cast<size_t>(d_o) * G);                 // proposal index
  c.take<int32_t>(2);                                             // moves, next rows
  c.take<int32_t>(static_cast<size_t>(d_o));                      // active rows
  c.take<int32_t>(static_cast<size_t>(d_o));                      // next active rows
  c.take<float>(static_cast<size_t>(d_i));                        // pair-term bound per column
  return c.used;
}

size_t gptq_ws(int64_t d_o, int64_t d_i) {
  Carver c(nullptr);
  c.take<uint32_t>(1);
  c.take<float>(static_cast<size_t>(d_o) * round_up(d_i, 4));   // W working copy
  c.take<float>(static_cast<size_t>(d_o) * 512);                 // E of a super-block
  c.take<float>(static_cast<size_t>(d_i) * round_up(d_i, 4));   // R^T
  c.take<uint32_t>(static_cast<size_t>(d_i));                    // permutation check
  c.used += rfactor_ws_bytes(d_i);
  return c.used;
}

size_t admm_ws(int64_t d_o, int64_t d_i, int64_t group, int64_t iters) {
  const int64_t ld = round_up(d_i, 4);
  const int64_t G = group > 0 ? d_i / group : 0;
  Carver c(nullptr);
  c.take<uint32_t>(1);
  c.take<float>(static_cast<size_t>(d_i) * ld);          // V^T
  for (int i = 0; i < 4; ++i) c.take<float>(static_cast<size_t>(d_o) * ld);   // P, M, T, W~
  c.take<float>(static_cast<size_t>(d_o) * d_i);         // U (when the caller passes none)
  c.take<float>(static_cast<size_t>(d_o) * G);           // lo_0
  c.take<float>(static_cast<size_t>(d_o) * G);           // hi_0
  c.take<float>(static_cast<size_t>(d_o) * G);           // s_0 scratch
  c.take<uint8_t>(static_cast<size_t>(d_o) * G);         // z_0 scratch
  c.take<float>(static_cast<size_t>(d_i));               // 1 / sigma
  c.take<double>(static_cast<size_t>(iters > 0 ? iters : 1) * admm_proj_blocks(G, d_o) * 2);
  return c.used;
}

}  // namespace

void set_error(const std::string& msg) { g_err = msg; }
const char* last_error() { return g_err.c_str(); }
int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}
int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QZ_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return QZ_OK;
}

}  // namespace qz

using namespace qz;

extern "C" {

const char* qz_last_error(void) { return qz::last_error(); }
int qz_abi_version(void) { return QZ_ABI_VERSION; }

// ------------------------------------------------------------------ Hessian
size_t qz_hessian_workspace(int64_t n, int64_t d_i, int32_t xt) {
  if (n < 0 || d_i < 1 || !valid_dtype(xt)) return 0;
  return hessian_ws_bytes(n, d_i, xt);
}

int qz_build_hessian(const void* X, int32_t xt, int64_t n, int64_t d_i, float damp, uint32_t flags,
                     float* H, float* diag, float* sigma, float* H_scaled, float* lambda_out,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(xt)) return fail(QZ_EINVAL, "build_hessian: bad dtype");
  if (n < 0 || d_i < 1) return fail(QZ_EINVAL, "build_hessian: need n >= 0 and d_i >= 1");
  if (!H || (n > 0 && !X)) return fail(QZ_EINVAL, "build_hessian: null pointer");
  if (H_scaled && H_scaled == H) return fail(QZ_EINVAL, "build_hessian: H_scaled must not alias H");
  if (H_scaled && (flags & QZ_H_NO_FINALIZE))
    return fail(QZ_EINVAL, "build_hessian: H_scaled needs a finalised H (no QZ_H_NO_FINALIZE)");
  if (!(damp >= 0.f) || !std::isfinite(damp)) return fail(QZ_EINVAL, "build_hessian: damp must be finite and >= 0");
  if (flags & ~(QZ_H_ACCUMULATE | QZ_H_NO_FINALIZE)) return fail(QZ_EINVAL, "build_hessian: unknown flags");
  const size_t need = hessian_ws_bytes(n, d_i, xt);
  if (ws_bytes < need || (need > 0 && !ws)) return fail(QZ_EWORKSPACE, "build_hessian: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(QZ_EWORKSPACE, "build_hessian: workspace must be 256-byte aligned");
  set_error("");
  return hessian_build(X, xt, n, d_i, damp, flags, H, diag, sigma, H_scaled, lambda_out, ws,
                       ws_bytes, stream);
}

// ------------------------------------------------------------------ RTN
size_t qz_rtn_workspace(int64_t d_o, int64_t d_i) {
  if (d_o < 0 || d_i < 1) return 0;
  return rtn_ws();
}

int qz_rtn(const void* W, int32_t wt, int64_t d_o, int64_t d_i, const qz_grid* grid,
           uint8_t* codes, float* scales, uint8_t* zeros, void* ws, size_t ws_bytes,
           hipStream_t stream) {
  if (!valid_dtype(wt)) return fail(QZ_EINVAL, "rtn: bad dtype");
  if (d_o < 0 || d_i < 1) return fail(QZ_EINVAL, "rtn: need d_o >= 0 and d_i >= 1");
  QZ_TRY(check_grid(grid, d_i));
  if (ws_bytes < rtn_ws() || !ws) return fail(QZ_EWORKSPACE, "rtn: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(QZ_EWORKSPACE, "rtn: workspace must be 256-byte aligned");
  if (d_o == 0) return QZ_OK;
  if (!W || !codes || !scales || !zeros) return fail(QZ_EINVAL, "rtn: null pointer");
  set_error("");
  return rtn_run(W, wt, d_o, d_i, grid, codes, scales, zeros, static_cast<uint32_t*>(ws), stream);
}

int qz_rtn_noalloc(const void* W, int32_t wt, int64_t d_o, int64_t d_i, const qz_grid* grid,
                   uint8_t* codes, float* scales, uint8_t* zeros, hipStream_t stream) {
  if (!valid_dtype(wt)) return fail(QZ_EINVAL, "rtn_noalloc: bad dtype");
  if (d_o < 0 || d_i < 1) return fail(QZ_EINVAL, "rtn_noalloc: need d_o >= 0 and d_i >= 1");
  QZ_TRY(check_grid(grid, d_i));
  // the scratch holds the status word only, so every size fits
  static_assert(kNoAllocScratchBytes >= sizeof(uint32_t), "scratch holds the status word");
  if (d_o == 0) return QZ_OK;
  if (!W || !codes || !scales || !zeros) return fail(QZ_EINVAL, "rtn_noalloc: null pointer");
  set_error("");
  uint32_t* flag = nullptr;
  QZ_TRY(noalloc_scratch(&flag));
  return rtn_run(W, wt, d_o, d_i, grid, codes, scales, zeros, flag, stream);
}

// ------------------------------------------------------------------ GPTQ
size_t qz_gptq_workspace(int64_t d_o, int64_t d_i, int32_t B) {
  if (d_o < 0 || d_i < 1 || B < 1 || B > 128) return 0;
  return gptq_ws(d_o, d_i);
}

static int gptq_blocks(float* Wf, int64_t ldw, float* E, int64_t lde, const float* Rt, int64_t ldr,
                       int64_t d_o, int64_t d_i, const qz_grid* grid, int32_t B,
                       const int32_t* perm, uint8_t* codes, int32_t* codes32, float* scales,
                       uint8_t* zeros, int64_t G, int64_t SB, hipStream_t stream);

// GPTQ with u8 codes clamped to the grid (codes) or unclamped int32 codes (codes32).
static int gptq_run(const float* H, const void* W_hat, int32_t wt, int64_t d_o, int64_t d_i,
                    const qz_grid* grid, int32_t B, const int32_t* perm, uint8_t* codes,
                    int32_t* codes32, float* scales, uint8_t* zeros, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  if (!valid_dtype(wt)) return fail(QZ_EINVAL, "gptq: bad dtype");
  if (d_o < 0 || d_i < 1) return fail(QZ_EINVAL, "gptq: need d_o >= 0 and d_i >= 1");
  if (B < 1 || B > 128) return fail(QZ_EINVAL, "gptq: block size B must be in 1..128");
  QZ_TRY(check_grid(grid, d_i));
  if (!H || (d_o > 0 && (!W_hat || (!codes && !codes32) || !scales || !zeros)))
    return fail(QZ_EINVAL, "gptq: null pointer");
  const size_t need = gptq_ws(d_o, d_i);
  if (ws_bytes < need || !ws) return fail(QZ_EWORKSPACE, "gptq: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(QZ_EWORKSPACE, "gptq: workspace must be 256-byte aligned");
  set_error("");

  // Two levels of lazy updates: blocks of B columns are grouped in super-blocks of up to
  // 512 columns; a block's E updates only the rest of its super-block, and after the
  // super-block one product with K = its width updates every later column (the same sums
  // as one update per block, in exact arithmetic, with far fewer passes over W).  A
  // block's E columns start 16-byte aligned inside the super-block's E only when B is a
  // multiple of 4; otherwise a super-block is one block.
  const int64_t SB = (B % 4 == 0) ? 512 / B : 1;   // blocks per super-block
  const int64_t ldw = round_up(d_i, 4), lde = 512, ldr = round_up(d_i, 4);
  const int64_t G = d_i / grid->group_size;
  Carver cv(ws);
  uint32_t* flag = cv.take<uint32_t>(1);
  float* Wf = cv.take<float>(static_cast<size_t>(d_o) * ldw);
  float* E = cv.take<float>(static_cast<size_t>(d_o) * lde);
  float* Rt = cv.take<float>(static_cast<size_t>(d_i) * ldr);
  uint32_t* counts = cv.take<uint32_t>(static_cast<size_t>(d_i));
  void* rws = cv.base + cv.used;

  QZ_TRY(launch_fill_u32(flag, 1, 0u, stream));
  if (perm) {
    // every later kernel indexes through perm: validate it first
    QZ_TRY(launch_check_perm(perm, d_i, counts, flag, stream));
    uint32_t hp = 0;
    QZ_TRY(read_flag(flag, stream, &hp));
    if (hp & FLAG_BADARG) return fail(QZ_EINVAL, "gptq: perm is not a permutation of 0..d_i-1");
  }
  // the grid and the fp32 copy of W need nothing from R: they run beside it
  hipStream_t side = stream;
  QZ_TRY(side_fork(stream, &side));
  if (d_o > 0) {
    ScopedTimer tm(K_GRID_RTN, side);
    if (!(grid->flags & QZ_GRID_CALLER))
      QZ_TRY(launch_grid_fit(W_hat, wt, d_o, d_i, grid->group_size, grid->bits, scales, zeros,
                             nullptr, nullptr, flag, side));
    QZ_TRY(launch_to_f32(W_hat, wt, d_o, d_i, perm, nullptr, Wf, ldw, flag, side));
  }
  {
    ScopedTimer tm(K_RFACTOR, stream);
    QZ_TRY(rfactor(H, d_i, perm, Rt, ldr, rws, flag, stream));
  }
  QZ_TRY(side_join(stream, side));
  // The factorisation's status is read once, at the end (the call's sync point): the
  // block loop is enqueued while R is still being formed, and after a failed
  // factorisation it only produces outputs that the error return leaves unspecified.
  if (d_o > 0) QZ_TRY(gptq_blocks(Wf, ldw, E, lde, Rt, ldr, d_o, d_i, grid, B, perm, codes,
                                  codes32, scales, zeros, G, SB, stream));
  uint32_t h = 0;
  QZ_TRY(read_flag(flag, stream, &h));   // SYNC: codes and grid are complete on return
  if (h & FLAG_NONFINITE) return fail(QZ_ENONFINITE, "gptq: non-finite H or W_hat");
  if (h & FLAG_NOTPD) return fail(QZ_ENOTPD, "gptq: H is not positive definite (increase damping)");
  return QZ_OK;
}

// The block loop of GPTQ (after R): per block the in-block kernel, then the lazy updates.
static int gptq_blocks(float* Wf, int64_t ldw, float* E, int64_t lde, const float* Rt, int64_t ldr,
                       int64_t d_o, int64_t d_i, const qz_grid* grid, int32_t B,
                       const int32_t* perm, uint8_t* codes, int32_t* codes32, float* scales,
                       uint8_t* zeros, int64_t G, int64_t SB, hipStream_t stream) {
  auto update = [&](const float* Eop, int64_t K, int64_t col0, int64_t ncols, int64_t rk) {
    // W[:, col0 : col0 + ncols] -= Eop[:, 0:K] R[rk : rk + K, col0 : col0 + ncols]
    GemmArgs g{};
    g.M = d_o;
    g.N = ncols;
    g.K = K;
    g.A = Eop;
    g.lda = lde;
    g.B = Rt + col0 * ldr + rk;   // row col0+n, columns rk.. : R[rk+k][col0+n]
    g.ldb = ldr;
    g.C = Wf + col0;
    g.ldc = ldw;
    ScopedTimer tm(K_GEMM_GPTQ, stream);
    return launch_gemm_nt(EPI_SUB, g, stream);
  };
  for (int64_t A = 0; A < d_i; A += SB * B) {
    const int64_t Aend = (A + SB * B < d_i) ? A + SB * B : d_i;
    for (int64_t a = A; a < Aend; a += B) {
      const int64_t b = (a + B < Aend) ? a + B : Aend;
      float* Eb = E + (a - A);
      {
        ScopedTimer tm(K_GPTQ_BLOCK, stream);
        QZ_TRY(launch_gptq_block(Wf, ldw, d_o, a, b, Rt, ldr, scales, zeros, G,
                                 grid->group_size, grid->bits, perm, Eb, lde, codes, codes32, d_i,
                                 stream));
      }
      if (b < Aend) QZ_TRY(update(Eb, b - a, b, Aend - b, a));          // rest of the super-block
    }
    if (Aend < d_i) QZ_TRY(update(E, Aend - A, Aend, d_i - Aend, A));   // every later column
  }
  return QZ_OK;
}

int qz_gptq(const float* H, const void* W_hat, int32_t wt, int64_t d_o, int64_t d_i,
            const qz_grid* grid, int32_t B, const int32_t* perm, uint8_t* codes, float* scales,
            uint8_t* zeros, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (d_o > 0 && !codes) return fail(QZ_EINVAL, "gptq: null pointer");
  return gptq_run(H, W_hat, wt, d_o, d_i, grid, B, perm, codes, nullptr, scales, zeros, ws,
                  ws_bytes, stream);
}

int qz_gptq_noclip(const float* H, const void* W_hat, int32_t wt, int64_t d_o, int64_t d_i,
                   const qz_grid* grid, int32_t B, const int32_t* perm, int32_t* codes,
                   float* scales, uint8_t* zeros, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (d_o > 0 && !codes) return fail(QZ_EINVAL, "gptq_noclip: null pointer");
  return gptq_run(H, W_hat, wt, d_o, d_i, grid, B, perm, nullptr, codes, scales, zeros, ws,
                  ws_bytes, stream);
}

// ------------------------------------------------------------------ orders, bound
size_t qz_order_workspace(int64_t d_i, int32_t kind) {
  if (d_i < 1 || (kind != QZ_ORDER_ACT && kind != QZ_ORDER_MIN_PIVOT)) return 0;
  Carver c(nullptr);
  c.take<uint32_t>(1);
  c.used += order_ws_bytes(d_i, kind);
  return c.used;
}

int qz_order(const float* H, int64_t d_i, int32_t kind, int32_t* perm, double* pivots, void* ws,
             size_t ws_bytes, hipStream_t stream) {
  if (d_i < 1) return fail(QZ_EINVAL, "order: d_i must be >= 1");
  if (d_i > 0x7fffffff) return fail(QZ_EINVAL, "order: d_i too large");
  if (kind != QZ_ORDER_ACT && kind != QZ_ORDER_MIN_PIVOT) return fail(QZ_EINVAL, "order: bad kind");
  if (!H || !perm) return fail(QZ_EINVAL, "order: null pointer");
  if (pivots && kind != QZ_ORDER_MIN_PIVOT)
    return fail(QZ_EINVAL, "order: pivots are returned by the min-pivot order only");
  const size_t need = qz_order_workspace(d_i, kind);
  if (ws_bytes < need || !ws) return fail(QZ_EWORKSPACE, "order: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(QZ_EWORKSPACE, "order: workspace must be 256-byte aligned");
  set_error("");
  Carver cv(ws);
  uint32_t* flag = cv.take<uint32_t>(1);
  void* rest = cv.base + cv.used;
  QZ_TRY(launch_fill_u32(flag, 1, 0u, stream));
  {
    ScopedTimer tm(K_ORDER, stream);
    if (kind == QZ_ORDER_ACT)
      QZ_TRY(order_act(H, d_i, perm, rest, flag, stream));
    else
      QZ_TRY(order_min_pivot(H, d_i, perm, pivots, rest, flag, stream));
  }
  uint32_t h = 0;
  QZ_TRY(read_flag(flag, stream, &h));
  if (h & FLAG_NONFINITE) return fail(QZ_ENONFINITE, "order: non-finite H");
  if (h & FLAG_NOTPD) return fail(QZ_ENOTPD, "order: H is not positive definite");
  return QZ_OK;
}

size_t qz_error_bound_workspace(int64_t d_o, int64_t d_i) {
  if (d_o < 0 || d_i < 1) return 0;
  Carver c(nullptr);
  c.take<uint32_t>(1);
  c.take<double>(1);                                   // total
  c.take<double>(static_cast<size_t>(d_i));            // D
  c.take<double>(static_cast<size_t>(d_o > 0 ? d_o : 1));   // row bounds when not given
  c.take<uint32_t>(static_cast<size_t>(d_i));          // permutation check
  c.used += rfactor_ws_bytes(d_i);
  return c.used;
}

int qz_error_bound(const float* H, int64_t d_i, const int32_t* perm, const float* scales,
                   int64_t d_o, int32_t group_size, double* row_bound, double* out_host, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  if (d_o < 0 || d_i < 1) return fail(QZ_EINVAL, "error_bound: need d_o >= 0 and d_i >= 1");
  if (group_size < 1 || d_i % group_size != 0)
    return fail(QZ_EINVAL, "error_bound: group_size must divide d_i");
  if (!H || (d_o > 0 && !scales)) return fail(QZ_EINVAL, "error_bound: null pointer");
  const size_t need = qz_error_bound_workspace(d_o, d_i);
  if (ws_bytes < need || !ws) return fail(QZ_EWORKSPACE, "error_bound: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(QZ_EWORKSPACE, "error_bound: workspace must be 256-byte aligned");
  set_error("");
  Carver cv(ws);
  uint32_t* flag = cv.take<uint32_t>(1);
  double* total = cv.take<double>(1);
  double* D = cv.take<double>(static_cast<size_t>(d_i));
  double* rows = cv.take<double>(static_cast<size_t>(d_o > 0 ? d_o : 1));
  uint32_t* counts = cv.take<uint32_t>(static_cast<size_t>(d_i));
  void* rws = cv.base + cv.used;
  QZ_TRY(launch_fill_u32(flag, 1, 0u, stream));
  if (perm) {
    QZ_TRY(launch_check_perm(perm, d_i, counts, flag, stream));
    uint32_t hp = 0;
    QZ_TRY(read_flag(flag, stream, &hp));
    if (hp & FLAG_BADARG)
      return fail(QZ_EINVAL, "error_bound: perm is not a permutation of 0..d_i-1");
  }
  {
    ScopedTimer tm(K_ORDER, stream);
    QZ_TRY(order_pivots(H, d_i, perm, D, rws, flag, stream));
    QZ_TRY(launch_error_bound(D, perm, scales, d_o, d_i, group_size, row_bound ? row_bound : rows,
                              total, stream));
  }
  uint32_t h = 0;
  QZ_TRY(read_flag(flag, stream, &h));
  if (h & FLAG_NONFINITE) return fail(QZ_ENONFINITE, "error_bound: non-finite H");
  if (h & FLAG_NOTPD) return fail(QZ_ENOTPD, "error_bound: H is not positive definite");
  if (out_host) {
    QZ_HIP(hipMemcpyAsync(out_host, total, sizeof(double), hipMemcpyDeviceToHost, stream));
    QZ_HIP(hipStreamSynchronize(stream));
  }
  return QZ_OK;
}

// ------------------------------------------------------------------ ADMM-Q
size_t qz_admmq_prepare_workspace(int64_t d_i) {
  if (d_i < 1) return 0;
  size_t b = 0;
  if (eig_ws_bytes(d_i, &b) != QZ_OK) return 0;
  return b;
}

int qz_admmq_prepare(const float* H, int64_t d_i, float* V, float* Lambda, float* sigma, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  if (d_i < 1) return fail(QZ_EINVAL, "admmq_prepare: d_i must be >= 1");
  if (!H || !V || !Lambda || !sigma) return fail(QZ_EINVAL, "admmq_prepare: null pointer");
  if (!ws) return fail(QZ_EWORKSPACE, "admmq_prepare: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(QZ_EWORKSPACE, "admmq_prepare: workspace must be 256-byte aligned");
  set_error("");
  ScopedTimer tm(K_EIG, stream);
  return eig_scaled(H, d_i, V, Lambda, sigma, ws, ws_bytes, stream);
}

size_t qz_admmq_workspace(int64_t d_o, int64_t d_i, int32_t group_size, int32_t iters) {
  if (d_o < 0 || d_i < 1 || group_size < 1 || d_i % group_size || iters < 0) return 0;
  return admm_ws(d_o, d_i, group_size, iters);
}

int qz_admmq(const float* V, const float* Lambda, const float* sigma, const void* W_hat, int32_t wt,
             int64_t d_o, int64_t d_i, const qz_grid* grid, const qz_admm* p, uint8_t* codes,
             float* scales, uint8_t* zeros, float* U, float* residuals, void* ws, size_t ws_bytes,
             hipStream_t stream) {
  if (!valid_dtype(wt)) return fail(QZ_EINVAL, "admmq: bad dtype");
  if (d_o < 0 || d_i < 1) return fail(QZ_EINVAL, "admmq: need d_o >= 0 and d_i >= 1");
  QZ_TRY(check_grid(grid, d_i));
  if (!p || p->struct_size < sizeof(qz_admm)) return fail(QZ_EINVAL, "admmq: params null or struct_size too small");
  const uint32_t known = QZ_ADMM_WARM_START | QZ_ADMM_REFRESH_UNCLAMPED | QZ_ADMM_REFRESH_FROM_Z |
                         QZ_ADMM_DUAL_NO_RESCALE;
  if (p->flags & ~known) return fail(QZ_EINVAL, "admmq: unknown flags");
  if ((p->flags & QZ_ADMM_REFRESH_UNCLAMPED) && (p->flags & QZ_ADMM_REFRESH_FROM_Z))
    return fail(QZ_EINVAL, "admmq: REFRESH_UNCLAMPED and REFRESH_FROM_Z are exclusive");
  if (p->iters < 0 || p->refresh_every < 0 || p->t0 < 0) return fail(QZ_EINVAL, "admmq: negative count");
  if (!(p->rho0 > 0.f) || !(p->gamma > 0.f) || !std::isfinite(p->rho0) || !std::isfinite(p->gamma))
    return fail(QZ_EINVAL, "admmq: rho0 and gamma must be finite and > 0");
  const bool warm = p->flags & QZ_ADMM_WARM_START;
  const bool caller_grid = grid->flags & QZ_GRID_CALLER;
  if (warm && !U) return fail(QZ_EINVAL, "admmq: WARM_START needs U");
  if (warm && caller_grid && p->refresh_every > 0)
    return fail(QZ_EINVAL, "admmq: WARM_START with a caller grid and refresh is not supported");
  if (!V || !Lambda || !sigma || (d_o > 0 && (!W_hat || !codes || !scales || !zeros)))
    return fail(QZ_EINVAL, "admmq: null pointer");
  const size_t need = admm_ws(d_o, d_i, grid->group_size, p->iters);
  if (ws_bytes < need || !ws) return fail(QZ_EWORKSPACE, "admmq: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(QZ_EWORKSPACE, "admmq: workspace must be 256-byte aligned");
  set_error("");
  if (d_o == 0) return QZ_OK;

  const int group = grid->group_size, bits = grid->bits;
  const int64_t ld = round_up(d_i, 4);
  const int64_t G = d_i / group;
  const int nblk = admm_proj_blocks(d_i / grid->group_size, d_o);
  Carver cv(ws);
  uint32_t* flag = cv.take<uint32_t>(1);
  float* Vt = cv.take<float>(static_cast<size_t>(d_i) * ld);
  float* P = cv.take<float>(static_cast<size_t>(d_o) * ld);
  float* M = cv.take<float>(static_cast<size_t>(d_o) * ld);
  float* T = cv.take<float>(static_cast<size_t>(d_o) * ld);
  float* Wt = cv.take<float>(static_cast<size_t>(d_o) * ld);
  float* Uws = cv.take<float>(static_cast<size_t>(d_o) * d_i);
  float* lo0 = cv.take<float>(static_cast<size_t>(d_o) * G);
  float* hi0 = cv.take<float>(static_cast<size_t>(d_o) * G);
  float* s0 = cv.take<float>(static_cast<size_t>(d_o) * G);
  uint8_t* z0 = cv.take<uint8_t>(static_cast<size_t>(d_o) * G);
  float* inv_sigma = cv.take<float>(static_cast<size_t>(d_i));
  double* partial = cv.take<double>(static_cast<size_t>(p->iters > 0 ? p->iters : 1) * nblk * 2);
  float* Ub = U ? U : Uws;

  QZ_TRY(launch_fill_u32(flag, 1, 0u, stream));
  QZ_TRY(launch_inverse_f32(sigma, d_i, inv_sigma, stream));
  QZ_TRY(launch_transpose_f32(V, d_i, d_i, d_i, Vt, ld, stream));
  // the static grid of W_hat: its range [lo_0, hi_0] bounds the refresh
  if (!caller_grid) {
    if (warm)
      QZ_TRY(launch_grid_fit(W_hat, wt, d_o, d_i, group, bits, s0, z0, lo0, hi0, flag, stream));
    else
      QZ_TRY(launch_grid_fit(W_hat, wt, d_o, d_i, group, bits, scales, zeros, lo0, hi0, flag, stream));
  } else {
    QZ_TRY(launch_range_of_grid(scales, zeros, d_o * G, bits, lo0, hi0, stream));
  }
  // P = W~_hat V Lambda with W~_hat = W_hat / Sigma (staged in T)
  QZ_TRY(launch_to_f32(W_hat, wt, d_o, d_i, nullptr, sigma, T, ld, flag, stream));
  {
    GemmArgs g{};
    g.M = d_o; g.N = d_i; g.K = d_i;
    g.A = T; g.lda = ld;
    g.B = Vt; g.ldb = ld;
    g.C = P; g.ldc = ld;
    g.colv = Lambda;
    ScopedTimer tm(K_GEMM_ADMM_SETUP, stream);
    QZ_TRY(launch_gemm_nt(EPI_COLSCALE, g, stream));
  }
  if (!warm) {
    QZ_TRY(launch_rtn(W_hat, wt, d_o, d_i, group, bits, scales, zeros, codes, stream));
    QZ_TRY(launch_fill_f32(Ub, d_o * d_i, 0.f, stream));
  }
  QZ_TRY(launch_admm_init_m(codes, scales, zeros, Ub, inv_sigma, d_o, d_i, group, M, ld, stream));

  int refresh_mode = 1;
  if (p->flags & QZ_ADMM_REFRESH_UNCLAMPED) refresh_mode = 2;
  if (p->flags & QZ_ADMM_REFRESH_FROM_Z) refresh_mode = 3;
  const int t0 = warm ? p->t0 : 0;
  for (int k = 0; k < p->iters; ++k) {
    const int t = t0 + k;
    const double rho = static_cast<double>(p->rho0) * std::pow(static_cast<double>(p->gamma), t);
    const double rho_next = rho * static_cast<double>(p->gamma);
    GemmArgs g1{};
    g1.M = d_o; g1.N = d_i; g1.K = d_i;
    g1.A = M; g1.lda = ld;
    g1.B = Vt; g1.ldb = ld;
    g1.C = T; g1.ldc = ld;
    g1.P = P; g1.ldp = ld;
    g1.colv = Lambda;
    g1.rho = static_cast<float>(rho);
    {
      ScopedTimer tm(K_GEMM_ADMM1, stream);
      QZ_TRY(launch_gemm_nt(EPI_ADMM1, g1, stream));
    }
    GemmArgs g2{};
    g2.M = d_o; g2.N = d_i; g2.K = d_i;
    g2.A = T; g2.lda = ld;
    g2.B = V; g2.ldb = d_i;
    g2.C = Wt; g2.ldc = ld;
    {
      ScopedTimer tm(K_GEMM_ADMM2, stream);
      QZ_TRY(launch_gemm_nt(EPI_STORE, g2, stream));
    }
    AdmmProj pr{};
    pr.Wt = Wt; pr.ldw = ld;
    pr.U = Ub;
    pr.M = M; pr.ldm = ld;
    pr.codes = codes;
    pr.scales = scales; pr.zeros = zeros;
    pr.lo0 = lo0; pr.hi0 = hi0;
    pr.sigma = sigma;
    pr.d_o = d_o; pr.d_i = d_i; pr.group = group; pr.bits = bits;
    pr.rho = static_cast<float>(rho);
    pr.rho_next = static_cast<float>(rho_next);
    pr.refresh = (p->refresh_every > 0 && t % p->refresh_every == 0) ? refresh_mode : 0;
    pr.rescale = (p->flags & QZ_ADMM_DUAL_NO_RESCALE) ? 0 : 1;
    pr.partial = partial + static_cast<int64_t>(k) * nblk * 2;
    ScopedTimer tm(K_ADMM_PROJECT, stream);
    QZ_TRY(launch_admm_project(pr, stream, inv_sigma));
  }
  QZ_TRY(launch_admm_residuals(partial, p->iters, nblk, residuals, flag, stream));
  uint32_t h = 0;
  QZ_TRY(read_flag(flag, stream, &h));
  if (h & FLAG_NONFINITE) return fail(QZ_ENONFINITE, "admmq: non-finite W_hat or iterate");
  return QZ_OK;
}

// ------------------------------------------------------------------ packing
int64_t qz_packed_words(int64_t cols, int32_t bits) {
  if (cols < 0 || bits < 1 || bits > 8) return -1;
  return ceil_div(cols * bits, 32);
}

int qz_pack(const uint8_t* codes, int64_t rows, int64_t cols, int32_t bits, uint32_t* out,
            hipStream_t stream) {
  if (rows < 0 || cols < 0 || bits < 1 || bits > 8) return fail(QZ_EINVAL, "pack: bad size or bits");
  if (rows * cols > 0 && (!codes || !out)) return fail(QZ_EINVAL, "pack: null pointer");
  set_error("");
  ScopedTimer tm(K_PACK, stream);
  return launch_pack(codes, rows, cols, bits, out, stream);
}

int qz_unpack(const uint32_t* in, int64_t rows, int64_t cols, int32_t bits, uint8_t* codes,
              hipStream_t stream) {
  if (rows < 0 || cols < 0 || bits < 1 || bits > 8) return fail(QZ_EINVAL, "unpack: bad size or bits");
  if (rows * cols > 0 && (!codes || !in)) return fail(QZ_EINVAL, "unpack: null pointer");
  set_error("");
  ScopedTimer tm(K_PACK, stream);
  return launch_unpack(in, rows, cols, bits, codes, stream);
}

// ------------------------------------------------------------------ objective
size_t qz_objective_workspace(int64_t d_o, int64_t d_i) {
  if (d_o < 0 || d_i < 1) return 0;
  return objective_ws(d_o, d_i);
}

// The objective of u8 codes (codes) or int32 codes (codes32).
static int objective_run(const float* H, const void* W_hat, int32_t wt, const uint8_t* codes,
                         const int32_t* codes32, const float* scales, const uint8_t* zeros,
                         int64_t d_o, int64_t d_i, int32_t group_size, double* row_f,
                         double* out_host, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(wt)) return fail(QZ_EINVAL, "objective: bad dtype");
  if (d_o < 0 || d_i < 1) return fail(QZ_EINVAL, "objective: need d_o >= 0 and d_i >= 1");
  if (group_size < 1 || d_i % group_size != 0)
    return fail(QZ_EINVAL, "objective: group_size must divide d_i");
  if (!H || (d_o > 0 && (!W_hat || (!codes && !codes32) || !scales || !zeros)))
    return fail(QZ_EINVAL, "objective: null pointer");
  const size_t need = objective_ws(d_o, d_i);
  if (ws_bytes < need || !ws) return fail(QZ_EWORKSPACE, "objective: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(QZ_EWORKSPACE, "objective: workspace must be 256-byte aligned");
  set_error("");
  if (d_o == 0) {
    if (out_host) *out_host = 0.0;
    return QZ_OK;
  }
  const int64_t ld = round_up(d_i, 4);
  const int tcols = gemm_tile_cols(d_i);
  Carver cv(ws);
  uint32_t* flag = cv.take<uint32_t>(1);
  float* D = cv.take<float>(static_cast<size_t>(d_o) * ld);
  double* dpart = cv.take<double>(static_cast<size_t>(d_o) * tcols);
  double* total = cv.take<double>(1);
  {
    ScopedTimer tm(K_OBJECTIVE, stream);
    QZ_TRY(launch_fill_u32(flag, 1, 0u, stream));
    if (codes32)
      QZ_TRY(launch_dequant_diff_i32(codes32, scales, zeros, W_hat, wt, d_o, d_i, group_size, D,
                                     ld, flag, stream));
    else
      QZ_TRY(launch_dequant_diff(codes, scales, zeros, W_hat, wt, d_o, d_i, group_size, D, ld,
                                 flag, stream));
    GemmArgs g{};
    g.M = d_o; g.N = d_i; g.K = d_i;
    g.A = D; g.lda = ld;
    g.B = H; g.ldb = d_i;          // H symmetric: row n of H is column n
    g.dpart = dpart;
    QZ_TRY(launch_gemm_nt(EPI_DOTROW, g, stream));
    QZ_TRY(launch_rowsum_half(dpart, d_o, tcols, row_f, total, stream));
  }
  if (out_host) {
    if (hipMemcpyAsync(out_host, total, sizeof(double), hipMemcpyDeviceToHost, stream) != hipSuccess)
      return fail(QZ_EHIP, "objective: copy of the result failed");
    uint32_t h = 0;
    QZ_TRY(read_flag(flag, stream, &h));   // synchronises the stream
    if (h & FLAG_NONFINITE) return fail(QZ_ENONFINITE, "objective: non-finite weight or grid");
  }
  return QZ_OK;
}

int qz_objective(const float* H, const void* W_hat, int32_t wt, const uint8_t* codes,
                 const float* scales, const uint8_t* zeros, int64_t d_o, int64_t d_i,
                 int32_t group_size, double* row_f, double* out_host, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  if (d_o > 0 && !codes) return fail(QZ_EINVAL, "objective: null pointer");
  return objective_run(H, W_hat, wt, codes, nullptr, scales, zeros, d_o, d_i, group_size, row_f,
                       out_host, ws, ws_bytes, stream);
}

int qz_objective_i32(const float* H, const void* W_hat, int32_t wt, const int32_t* codes,
                     const float* scales, const uint8_t* zeros, int64_t d_o, int64_t d_i,
                     int32_t group_size, double* row_f, double* out_host, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  if (d_o > 0 && !codes) return fail(QZ_EINVAL, "objective: null pointer");
  return objective_run(H, W_hat, wt, nullptr, codes, scales, zeros, d_o, d_i, group_size, row_f,
                       out_host, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ local search
size_t qz_local_search_workspace(int64_t d_o, int64_t d_i, int32_t group_size) {
  if (d_o < 0 || d_i < 1 || group_size < 1 || d_i % group_size != 0) return 0;
  return lsearch_ws(d_o, d_i, group_size);
}

int qz_local_search(const float* H, const void* W_hat, int32_t wt, int64_t d_o, int64_t d_i,
                    const qz_grid* grid, const float* scales, const uint8_t* zeros,
                    uint8_t* codes, int32_t max_steps, int32_t* moves_host, int32_t* steps_host,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(wt)) return fail(QZ_EINVAL, "local_search: bad dtype");
  if (d_o < 0 || d_i < 1) return fail(QZ_EINVAL, "local_search: need d_o >= 0 and d_i >= 1");
  QZ_TRY(check_grid(grid, d_i));
  const int group = grid->group_size, bits = grid->bits;
  if (group > ls_max_group())
    return fail(QZ_EINVAL, "local_search: groups of at most 128 columns are supported");
  if (max_steps < 0) return fail(QZ_EINVAL, "local_search: max_steps must be >= 0");
  const int64_t G = d_i / group;
  if (ls_accept_lds(G) > 65536) return fail(QZ_EINVAL, "local_search: too many groups per row");
  if (!H || (d_o > 0 && (!W_hat || !codes || !scales || !zeros)))
    return fail(QZ_EINVAL, "local_search: null pointer");
  const size_t need = lsearch_ws(d_o, d_i, group);
  if (ws_bytes < need || !ws) return fail(QZ_EWORKSPACE, "local_search: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(QZ_EWORKSPACE, "local_search: workspace must be 256-byte aligned");
  set_error("");
  if (steps_host) *steps_host = 0;
  if (d_o == 0 || max_steps == 0) return QZ_OK;
  const int64_t ld = round_up(d_i, 4);
  Carver cv(ws);
  uint32_t* flag = cv.take<uint32_t>(1);
  float* D = cv.take<float>(static_cast<size_t>(d_o) * ld);
  float* Gm = cv.take<float>(static_cast<size_t>(d_o) * ld);
  float* best_df = cv.take<float>(static_cast<size_t>(d_o) * G);
  int32_t* best_idx = cv.take<int32_t>(static_cast<size_t>(d_o) * G);
  int32_t* counters = cv.take<int32_t>(2);
  int32_t* act = cv.take<int32_t>(static_cast<size_t>(d_o));
  int32_t* next = cv.take<int32_t>(static_cast<size_t>(d_o));
  float* hmax = cv.take<float>(static_cast<size_t>(d_i));
  QZ_TRY(launch_fill_u32(flag, 1, 0u, stream));
  {
    // the gradient of every row once, on the matrix cores; afterwards it is updated
    // row by row with the accepted moves
    ScopedTimer tm(K_LS_GRADIENT, stream);
    QZ_TRY(launch_dequant_diff(codes, scales, zeros, W_hat, wt, d_o, d_i, group, D, ld, flag,
                               stream));
    GemmArgs g{};
    g.M = d_o; g.N = d_i; g.K = d_i;
    g.A = D; g.lda = ld;
    g.B = H; g.ldb = d_i;      // H symmetric
    g.C = Gm; g.ldc = ld;
    QZ_TRY(launch_gemm_nt(EPI_STORE, g, stream));
    QZ_TRY(launch_ls_iota(act, d_o, stream));
    QZ_TRY(launch_ls_hmax(H, d_i, group, hmax, stream));
  }
  int64_t n_act = d_o;
  int steps = 0;
  for (int t = 0; t < max_steps; ++t) {
    {
      ScopedTimer tm(K_LS_PROPOSE, stream);
      QZ_TRY(launch_ls_propose(Gm, ld, H, d_i, hmax, codes, scales, group, bits, act, n_act,
                               best_df, best_idx, stream));
    }
    {
      ScopedTimer tm(K_LS_ACCEPT, stream);
      QZ_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(counters), 2, 0u, stream));
      QZ_TRY(launch_ls_accept(H, d_i, codes, scales, group, best_df, best_idx, act, n_act, Gm, ld,
                              t + 1 < max_steps, next, counters, stream));
    }
    int32_t host_counters[2] = {0, 0};
    QZ_HIP(hipMemcpyAsync(host_counters, counters, sizeof(host_counters), hipMemcpyDeviceToHost,
                          stream));
    QZ_HIP(hipStreamSynchronize(stream));
    if (moves_host) moves_host[t] = host_counters[0];
    if (host_counters[0] == 0) break;
    steps = t + 1;
    n_act = host_counters[1];
    int32_t* tmp = act;
    act = next;
    next = tmp;
  }
  if (steps_host) *steps_host = steps;
  uint32_t h = 0;
  QZ_TRY(read_flag(flag, stream, &h));
  if (h & FLAG_NONFINITE) return fail(QZ_ENONFINITE, "local_search: non-finite weight or grid");
  return QZ_OK;
}

}  // extern "C"
