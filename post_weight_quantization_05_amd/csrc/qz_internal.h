// Internal declarations shared by the libqz translation units (host launchers and
// device helpers).  Not part of the public ABI (include/qz.h is).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "qz.h"

namespace qz {

// ------------------------------------------------------------------ errors
void set_error(const std::string& msg);
const char* last_error();

struct Status {
  int code = QZ_OK;
  bool ok() const { return code == QZ_OK; }
};

int fail(int code, const std::string& msg);

#define QZ_HIP(expr)                                                              \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess)                                                         \
      return ::qz::fail(QZ_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

#define QZ_TRY(expr)                 \
  do {                               \
    int r_ = (expr);                 \
    if (r_ != QZ_OK) return r_;      \
  } while (0)

// Launch-error check after a kernel launch.
int check_launch(const char* what);

// ------------------------------------------------------------------ timing
enum KernelKind : int {
  K_HESSIAN_GRAM = 0,
  K_HESSIAN_FINISH,
  K_RFACTOR,
  K_GPTQ_BLOCK,
  K_GEMM_GPTQ,
  K_GEMM_ADMM_SETUP,
  K_GEMM_ADMM1,
  K_GEMM_ADMM2,
  K_ADMM_PROJECT,
  K_ADMM_OTHER,
  K_GRID_RTN,
  K_PACK,
  K_EIG,
  K_OBJECTIVE,
  K_LS_GRADIENT,
  K_LS_PROPOSE,
  K_LS_ACCEPT,
  K_ORDER,
  K_KIND_COUNT
};
// Records an event pair around the enclosed launches when timing is enabled.
class ScopedTimer {
 public:
  ScopedTimer(int kind, hipStream_t s);
  ~ScopedTimer();
  ScopedTimer(const ScopedTimer&) = delete;
  ScopedTimer& operator=(const ScopedTimer&) = delete;

 private:
  int kind_;
  hipStream_t s_;
  hipEvent_t b_ = nullptr, e_ = nullptr;
};

// ------------------------------------------------------------------ sizes
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Carves aligned sub-buffers out of a caller workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used = align256(used + count * sizeof(T));
    return p;
  }
};

// Device status word bits (written with integer atomicOr through vector memory).
enum : uint32_t { FLAG_NONFINITE = 1u, FLAG_NOTPD = 2u, FLAG_BADARG = 4u };

// ------------------------------------------------------------------ device helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <int WT>
__device__ __forceinline__ float load_w(const void* p, int64_t i) {
  if constexpr (WT == QZ_BF16)
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else
    return static_cast<const float*>(p)[i];
}

// code = clamp(rint(x / s) + z, 0, maxq) with IEEE fp32 division and
// round-half-to-even; identical to the fp32 definition of the grid.
__device__ __forceinline__ float quant_code(float x, float s, float z, float maxq) {
  float u = __builtin_rintf(x / s) + z;
  return fminf(fmaxf(u, 0.0f), maxq);
}

// ------------------------------------------------------------------ launchers
// grid / rtn / pack (k_grid.hip)
int launch_grid_fit(const void* W, int wt, int64_t rows, int64_t cols, int group, int bits,
                    float* scales, uint8_t* zeros, float* lo0, float* hi0, uint32_t* flag,
                    hipStream_t s);
int launch_rtn(const void* W, int wt, int64_t rows, int64_t cols, int group, int bits,
               const float* scales, const uint8_t* zeros, uint8_t* codes, hipStream_t s);
int launch_pack(const uint8_t* codes, int64_t rows, int64_t cols, int bits, uint32_t* out,
                hipStream_t s);
int launch_unpack(const uint32_t* in, int64_t rows, int64_t cols, int bits, uint8_t* codes,
                  hipStream_t s);
// W_hat (any dtype) -> fp32 [rows x ldo], optional column gather (out col j = in col perm[j])
// and optional per-column division by div[c]; sets FLAG_NONFINITE on a non-finite value.
int launch_to_f32(const void* W, int wt, int64_t rows, int64_t cols, const int32_t* perm,
                  const float* div, float* out, int64_t ldo, uint32_t* flag, hipStream_t s);
int launch_check_finite_f32(const float* p, int64_t n, uint32_t* flag, hipStream_t s);
// D = s (C - z) - W_hat  (fp32 [rows x ldo], zero padding columns up to ldo); sets
// FLAG_NONFINITE on a non-finite value
int launch_dequant_diff(const uint8_t* codes, const float* scales, const uint8_t* zeros,
                        const void* W, int wt, int64_t rows, int64_t cols, int group, float* out,
                        int64_t ldo, uint32_t* flag, hipStream_t s);
// the same for int32 codes (unclamped GPTQ codes)
int launch_dequant_diff_i32(const int32_t* codes, const float* scales, const uint8_t* zeros,
                            const void* W, int wt, int64_t rows, int64_t cols, int group,
                            float* out, int64_t ldo, uint32_t* flag, hipStream_t s);
// row_f[r] = 0.5 * sum_t dpart[r][t]; total = sum_r row_f[r] (fixed order, one workgroup)
int launch_rowsum_half(const double* dpart, int64_t rows, int64_t tcols, double* row_f,
                       double* total, hipStream_t s);
// Sets FLAG_BADARG unless perm[0..d) is a permutation of 0..d-1 (counts: d ints of scratch).
int launch_check_perm(const int32_t* perm, int64_t d, uint32_t* counts, uint32_t* flag, hipStream_t s);

// fp32 matrix-core GEMM  C (epilogue)= A[M x K] * B[N x K]^T  (k_gemm.hip)
enum GemmEpi : int {
  EPI_STORE = 0,     // C = acc
  EPI_SUB = 1,       // C = C - A B (accumulated from C with A negated)
  EPI_COLSCALE = 2,  // C = acc * colv[n]
  EPI_ADMM1 = 3,     // C = (P + rho * acc) / (colv[n] + rho)
  EPI_ADD = 4,       // C = C + acc
  EPI_DOTROW = 5,    // dpart[m][tile column] = sum over the tile's columns of acc * A[m][n]
                     // (C unused; needs N == K so that A[m][n] exists)
};
struct GemmArgs {
  int64_t M, N, K;
  const float* A; int64_t lda;
  const float* B; int64_t ldb;
  float* C; int64_t ldc;
  const float* P; int64_t ldp;   // EPI_ADMM1
  const float* colv;             // EPI_COLSCALE / EPI_ADMM1
  float rho;
  double* dpart;                 // EPI_DOTROW: [M x ceil(N / 128)]
};
int gemm_tile_cols(int64_t N);   // ceil(N / 128): tile columns of the GEMM
int launch_gemm_nt(int epi, const GemmArgs& a, hipStream_t s);

// pairwise-swap local search (k_lsearch.hip)
int ls_max_group();
size_t ls_accept_lds(int64_t G);
int launch_ls_iota(int32_t* p, int64_t n, hipStream_t s);   // p[i] = i
// hmax[c] = max |H[c][k]| over the other columns k of c's group
int launch_ls_hmax(const float* H, int64_t d_i, int group, float* hmax, hipStream_t s);
// best move per (act[a], group) for a < n_act -> best_df / best_idx [rows x G]
int launch_ls_propose(const float* Gm, int64_t ldg, const float* H, int64_t d_i,
                      const float* hmax, const uint8_t* codes, const float* scales, int group,
                      int bits, const int32_t* act, int64_t n_act, float* best_df,
                      int32_t* best_idx, hipStream_t s);
// accept, apply, append moved rows to next_act (counters[0] += moves, counters[1] = slots)
// and, when update, add the accepted moves' H rows to the gradient rows
int launch_ls_accept(const float* H, int64_t d_i, uint8_t* codes, const float* scales, int group,
                     const float* best_df, const int32_t* best_idx, const int32_t* act,
                     int64_t n_act, float* Gm, int64_t ldg, bool update, int32_t* next_act,
                     int32_t* counters, hipStream_t s);

// bf16 Hessian (k_hessian.hip)
size_t hessian_ws_bytes(int64_t n, int64_t d, int xt);
int hessian_build(const void* X, int xt, int64_t n, int64_t d, float damp, uint32_t flags,
                  float* H, float* diag, float* sigma, float* H_scaled, float* lambda_out,
                  void* ws, size_t ws_bytes, hipStream_t s);

// orders and the error bound (k_order.hip)
size_t order_ws_bytes(int64_t n, int kind);
int order_act(const float* H, int64_t n, int32_t* perm, void* ws, uint32_t* flag, hipStream_t s);
int order_min_pivot(const float* H, int64_t n, int32_t* perm, double* pivots, void* ws,
                    uint32_t* flag, hipStream_t s);
// row_bound[r] = 1/8 sum_j D[j] s(r, perm[j] / group)^2; *total = fixed-order row sum
int launch_error_bound(const double* D, const int32_t* perm, const float* scales, int64_t d_o,
                       int64_t d_i, int group, double* row_bound, double* total, hipStream_t s);

// fp64 Cholesky / inverse factor (k_chol.hip)
size_t rfactor_ws_bytes(int64_t d);
// Rt (lower, row-major, ld ldr) = R^T where R is upper with R^T R = Hp^{-1},
// Hp = H[perm][:, perm] (perm may be null).  Sets FLAG_NOTPD / FLAG_NONFINITE.
int rfactor(const float* H, int64_t d, const int32_t* perm, float* Rt, int64_t ldr, void* ws,
            uint32_t* flag, hipStream_t s);
// D[j] (fp64, [d]) = LDL pivot of the column quantized j-th in the order perm (null =
// natural): the diagonal of Hp reordered so the column quantized last is eliminated
// first, i.e. 1 / R_jj^2 of GPTQ's factor.  Same workspace and flags as rfactor.
int order_pivots(const float* H, int64_t d, const int32_t* perm, double* D, void* ws,
                 uint32_t* flag, hipStream_t s);
// A stream for work beside the factorisation (waits for what `s` holds so far; `s`
// itself without side streams), and the join back into `s`.
int side_fork(hipStream_t s, hipStream_t* side);
int side_join(hipStream_t s, hipStream_t side);

// GPTQ in-block column kernel (k_gptq.hip)
int launch_gptq_block(float* W, int64_t ldw, int64_t d_o, int64_t a, int64_t b, const float* Rt,
                      int64_t ldr, const float* scales, const uint8_t* zeros, int64_t n_groups,
                      int group, int bits, const int32_t* perm, float* E, int64_t lde,
                      uint8_t* codes, int32_t* codes32, int64_t d_i, hipStream_t s);

// ADMM kernels (k_admm.hip)
struct AdmmProj {
  const float* Wt; int64_t ldw;     // continuous iterate (scaled space)
  float* U;                          // [d_o x d_i] dense
  float* M; int64_t ldm;             // next GEMM input D~ - U
  uint8_t* codes;                    // [d_o x d_i]
  float* scales; uint8_t* zeros;     // [d_o x G]
  const float* lo0; const float* hi0;
  const float* sigma;
  int64_t d_o, d_i; int group, bits;
  float rho, rho_next;
  int refresh;                       // 0 none, 1 clamped, 2 unclamped, 3 from-z (clamped)
  int rescale;                       // 1: U *= rho/rho_next
  double* partial;                   // [nblocks x 2] for this iteration
};
int admm_proj_blocks(int64_t G, int64_t d_o);   // workgroups of a projection launch (partials per iteration)
int launch_admm_project(const AdmmProj& p, hipStream_t s, const float* inv_sigma);
int launch_admm_init_m(const uint8_t* codes, const float* scales, const uint8_t* zeros,
                       const float* U, const float* sigma, int64_t d_o, int64_t d_i, int group,
                       float* M, int64_t ldm, hipStream_t s);
int launch_admm_residuals(const double* partial, int iters, int nblocks, float* residuals,
                          uint32_t* flag, hipStream_t s);
int launch_transpose_f32(const float* in, int64_t rows, int64_t cols, int64_t ldi, float* out,
                         int64_t ldo, hipStream_t s);
int launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
int launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
int launch_inverse_f32(const float* x, int64_t n, float* y, hipStream_t s);
int launch_range_of_grid(const float* scales, const uint8_t* zeros, int64_t n, int bits,
                         float* lo0, float* hi0, hipStream_t s);
int launch_copy_bytes(const void* src, int64_t n, void* dst, hipStream_t s);

// eigendecomposition of Sigma H Sigma (k_eig.hip): workspace bytes (asks the solver library
// for its scratch size once per size), and the decomposition in the caller's workspace
int eig_ws_bytes(int64_t d, size_t* bytes);
int eig_scaled(const float* H, int64_t d, float* V, float* Lambda, float* sigma, void* ws,
               size_t ws_bytes, hipStream_t s);

}  // namespace qz
