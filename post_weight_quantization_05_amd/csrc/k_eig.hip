// Eigendecomposition of the scaled Hessian for the ADMM-Q W-update (ADMM-Q summary,
// 2. key components: the W-update is evaluated through an eigendecomposition of H,
// here of H~ = Sigma H Sigma with Sigma = diag(H)^(-1/2)).  A one-time set-up step:
// H~ is formed in fp64 on the device and handed to rocSOLVER's divide-and-conquer
// symmetric eigensolver (a library call standing in for host LAPACK); V and Lambda
// come back in fp32.  Every device byte the call uses -- the fp64 matrix, the
// eigenvalue and off-diagonal vectors, the solver's own scratch -- comes from the
// caller's workspace: the solver's scratch size is asked of the library once per
// size (its device-memory size query) and handed to it with rocblas_set_workspace.
// The rocBLAS handle is created once per host thread and device and kept.
#include <rocblas/rocblas.h>
#include <rocsolver/rocsolver.h>

#include <vector>

#include "qz_internal.h"

namespace qz {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void sigma_kernel(const float* __restrict__ H, int64_t d,
                                                         float* __restrict__ sigma,
                                                         double* __restrict__ sig64,
                                                         uint32_t* __restrict__ flag) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < d;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float h = H[i * d + i];
    if (!(h > 0.f) || !__builtin_isfinite(h)) atomicOr(flag, FLAG_NONFINITE);
    sigma[i] = 1.0f / sqrtf(h);
    sig64[i] = 1.0 / sqrt(static_cast<double>(h));
  }
}

__global__ __launch_bounds__(kThreads) void scale_kernel(const float* __restrict__ H, int64_t d,
                                                         const double* __restrict__ sig64,
                                                         double* __restrict__ A,
                                                         uint32_t* __restrict__ flag) {
  bool bad = false;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < d * d;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / d, j = e % d;
    const float h = H[e];
    bad |= !__builtin_isfinite(h);
    A[e] = static_cast<double>(h) * sig64[i] * sig64[j];
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, FLAG_NONFINITE);
}

// A is column-major from the solver: eigenvector k is column k, A[j + k d] = V[j][k].
__global__ __launch_bounds__(kThreads) void export_kernel(const double* __restrict__ A,
                                                          const double* __restrict__ D, int64_t d,
                                                          float* __restrict__ V,
                                                          float* __restrict__ Lambda) {
  __shared__ double t[32][33];
  const int64_t k0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) {
    const int64_t k = k0 + r, j = j0 + tx;     // contiguous in j within column k
    t[r][tx] = (k < d && j < d) ? A[j + k * d] : 0.0;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t j = j0 + r, k = k0 + tx;     // V row j, contiguous in k
    if (j < d && k < d) V[j * d + k] = static_cast<float>(t[tx][r]);
  }
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int64_t i = threadIdx.x; i < d; i += blockDim.x) Lambda[i] = static_cast<float>(D[i]);
}

inline unsigned grid_for(int64_t n) {
  int64_t b = ceil_div(n, kThreads * 4);
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return static_cast<unsigned>(b);
}

struct SolverHandle {
  int device = -1;
  rocblas_handle h = nullptr;
};

// One rocBLAS handle per host thread and device, created on first use and kept (like the
// R factor's side streams): creating a handle per call would cost more than a small solve.
int solver_handle(rocblas_handle* out) {
  int dev = 0;
  QZ_HIP(hipGetDevice(&dev));
  thread_local std::vector<SolverHandle> cache;
  for (const SolverHandle& c : cache)
    if (c.device == dev) {
      *out = c.h;
      return QZ_OK;
    }
  SolverHandle c;
  c.device = dev;
  if (rocblas_create_handle(&c.h) != rocblas_status_success)
    return fail(QZ_ESOLVER, "admmq_prepare: rocblas_create_handle failed");
  cache.push_back(c);
  *out = c.h;
  return QZ_OK;
}

// Scratch bytes rocsolver_dsyevd needs for an n x n problem (the library's size-query
// mode: nothing runs and no pointer is dereferenced, but the argument checks want
// non-null pointers, so host dummies stand in).
int solver_scratch(rocblas_handle h, int64_t n, size_t* bytes) {
  static double dummy[4];
  static rocblas_int dummy_info;
  if (rocblas_start_device_memory_size_query(h) != rocblas_status_success)
    return fail(QZ_ESOLVER, "admmq_prepare: solver size query failed to start");
  const rocblas_status st = rocsolver_dsyevd(h, rocblas_evect_original, rocblas_fill_upper,
                                             static_cast<rocblas_int>(n), dummy,
                                             static_cast<rocblas_int>(n), dummy, dummy,
                                             &dummy_info);
  size_t sz = 0;
  const rocblas_status st2 = rocblas_stop_device_memory_size_query(h, &sz);
  if ((st != rocblas_status_success && st != rocblas_status_size_increased &&
       st != rocblas_status_size_unchanged) ||
      st2 != rocblas_status_success)
    return fail(QZ_ESOLVER, "admmq_prepare: solver size query failed (" + std::to_string(int(st)) +
                                ", " + std::to_string(int(st2)) + ")");
  *bytes = sz;
  return QZ_OK;
}

struct EigLayout {
  size_t A, D, E, sig64, info, flag, scratch, total;
};

EigLayout eig_layout(int64_t d, size_t scratch) {
  EigLayout l;
  Carver c(nullptr);
  l.A = c.used;     c.take<double>(static_cast<size_t>(d) * d);
  l.D = c.used;     c.take<double>(static_cast<size_t>(d));
  l.E = c.used;     c.take<double>(static_cast<size_t>(d));
  l.sig64 = c.used; c.take<double>(static_cast<size_t>(d));
  l.info = c.used;  c.take<rocblas_int>(1);
  l.flag = c.used;  c.take<uint32_t>(1);
  l.scratch = c.used;
  l.total = align256(c.used + scratch);
  return l;
}

}  // namespace

int eig_ws_bytes(int64_t d, size_t* bytes) {
  if (d > 46340) return fail(QZ_EINVAL, "admmq_prepare: d_i too large for the eigensolver");
  rocblas_handle h = nullptr;
  QZ_TRY(solver_handle(&h));
  size_t scratch = 0;
  QZ_TRY(solver_scratch(h, d, &scratch));
  *bytes = eig_layout(d, scratch).total;
  return QZ_OK;
}

int eig_scaled(const float* H, int64_t d, float* V, float* Lambda, float* sigma, void* ws,
               size_t ws_bytes, hipStream_t s) {
  if (d > 46340) return fail(QZ_EINVAL, "admmq_prepare: d_i too large for the eigensolver");
  rocblas_handle handle = nullptr;
  QZ_TRY(solver_handle(&handle));
  size_t scratch = 0;
  QZ_TRY(solver_scratch(handle, d, &scratch));
  const EigLayout l = eig_layout(d, scratch);
  if (!ws || ws_bytes < l.total) return fail(QZ_EWORKSPACE, "admmq_prepare: workspace too small");
  char* base = static_cast<char*>(ws);
  double* A = reinterpret_cast<double*>(base + l.A);
  double* D = reinterpret_cast<double*>(base + l.D);
  double* E = reinterpret_cast<double*>(base + l.E);
  double* sig64 = reinterpret_cast<double*>(base + l.sig64);
  rocblas_int* info = reinterpret_cast<rocblas_int*>(base + l.info);
  uint32_t* flag = reinterpret_cast<uint32_t*>(base + l.flag);

  QZ_TRY(launch_fill_u32(flag, 1, 0u, s));
  sigma_kernel<<<grid_for(d), kThreads, 0, s>>>(H, d, sigma, sig64, flag);
  QZ_TRY(check_launch("eig.sigma"));
  scale_kernel<<<grid_for(d * d), kThreads, 0, s>>>(H, d, sig64, A, flag);
  QZ_TRY(check_launch("eig.scale"));
  uint32_t hflag = 0;
  QZ_HIP(hipMemcpyAsync(&hflag, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  QZ_HIP(hipStreamSynchronize(s));
  if (hflag & FLAG_NONFINITE)
    return fail(QZ_ENONFINITE, "admmq_prepare: H has a non-finite entry or a non-positive diagonal");

  // the solver runs on the caller's stream, in the caller's memory; the handle is
  // detached from that memory again before the call returns
  if (rocblas_set_stream(handle, s) != rocblas_status_success ||
      rocblas_set_workspace(handle, scratch ? base + l.scratch : nullptr, scratch) !=
          rocblas_status_success)
    return fail(QZ_ESOLVER, "admmq_prepare: could not attach the solver workspace");
  const rocblas_status st = rocsolver_dsyevd(handle, rocblas_evect_original, rocblas_fill_upper,
                                             static_cast<rocblas_int>(d), A,
                                             static_cast<rocblas_int>(d), D, E, info);
  int hinfo = 0;
  const hipError_t ec = hipMemcpyAsync(&hinfo, info, sizeof(int), hipMemcpyDeviceToHost, s);
  const hipError_t es = hipStreamSynchronize(s);
  rocblas_set_workspace(handle, nullptr, 0);
  if (st != rocblas_status_success)
    return fail(QZ_ESOLVER, "admmq_prepare: rocsolver_dsyevd status " + std::to_string(int(st)));
  if (ec != hipSuccess || es != hipSuccess) return fail(QZ_EHIP, "admmq_prepare: sync failed");
  if (hinfo != 0)
    return fail(QZ_ESOLVER, "admmq_prepare: eigensolver did not converge (info " +
                                std::to_string(hinfo) + ")");
  dim3 grid(static_cast<unsigned>(ceil_div(d, 32)), static_cast<unsigned>(ceil_div(d, 32)));
  export_kernel<<<grid, kThreads, 0, s>>>(A, D, d, V, Lambda);
  QZ_TRY(check_launch("eig.export"));
  // the workspace holds the fp64 factors until the export has read them
  QZ_HIP(hipStreamSynchronize(s));
  return QZ_OK;
}

}  // namespace qz
