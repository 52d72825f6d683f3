// Eigendecomposition of the scaled Hessian for the ADMM-Q W-update (ADMM-Q summary,
// 2. key components: the W-update is evaluated through an eigendecomposition of H,
// here of H~ = Sigma H Sigma with Sigma = diag(H)^(-1/2)).  A one-time set-up step:
// H~ is formed in fp64 on the device and handed to rocSOLVER's divide-and-conquer
// symmetric eigensolver (a library call standing in for host LAPACK); V and Lambda
// come back in fp32.
#include <rocblas/rocblas.h>
#include <rocsolver/rocsolver.h>

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

}  // namespace

int eig_scaled(const float* H, int64_t d, float* V, float* Lambda, float* sigma, hipStream_t s) {
  if (d > 46340) return fail(QZ_EINVAL, "admmq_prepare: d_i too large for the eigensolver");
  double* A = nullptr;
  double* D = nullptr;
  double* E = nullptr;
  double* sig64 = nullptr;
  int* info = nullptr;
  uint32_t* flag = nullptr;
  rocblas_handle handle = nullptr;
  int rc = QZ_OK;
  auto cleanup = [&]() {
    if (handle) rocblas_destroy_handle(handle);
    (void)hipFree(A);
    (void)hipFree(D);
    (void)hipFree(E);
    (void)hipFree(sig64);
    (void)hipFree(info);
    (void)hipFree(flag);
  };
  do {
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&A), sizeof(double) * d * d);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&D), sizeof(double) * d);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&E), sizeof(double) * d);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&sig64), sizeof(double) * d);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&info), sizeof(int));
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&flag), sizeof(uint32_t));
    if (e != hipSuccess) {
      rc = fail(QZ_EHIP, std::string("admmq_prepare: device allocation failed: ") +
                             hipGetErrorName(e) + " " + hipGetErrorString(e));
      break;
    }
    if ((rc = launch_fill_u32(flag, 1, 0u, s)) != QZ_OK) break;
    sigma_kernel<<<grid_for(d), kThreads, 0, s>>>(H, d, sigma, sig64, flag);
    if ((rc = check_launch("eig.sigma")) != QZ_OK) break;
    scale_kernel<<<grid_for(d * d), kThreads, 0, s>>>(H, d, sig64, A, flag);
    if ((rc = check_launch("eig.scale")) != QZ_OK) break;
    uint32_t hflag = 0;
    if (hipMemcpyAsync(&hflag, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
      rc = fail(QZ_EHIP, "admmq_prepare: sync failed");
      break;
    }
    if (hflag & FLAG_NONFINITE) {
      rc = fail(QZ_ENONFINITE, "admmq_prepare: H has a non-finite entry or a non-positive diagonal");
      break;
    }
    if (rocblas_create_handle(&handle) != rocblas_status_success ||
        rocblas_set_stream(handle, s) != rocblas_status_success) {
      rc = fail(QZ_ESOLVER, "admmq_prepare: rocblas handle");
      break;
    }
    rocblas_status st = rocsolver_dsyevd(handle, rocblas_evect_original, rocblas_fill_upper,
                                         static_cast<rocblas_int>(d), A, static_cast<rocblas_int>(d),
                                         D, E, info);
    if (st != rocblas_status_success) {
      rc = fail(QZ_ESOLVER, "admmq_prepare: rocsolver_dsyevd status " + std::to_string(int(st)));
      break;
    }
    int hinfo = 0;
    if (hipMemcpyAsync(&hinfo, info, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
      rc = fail(QZ_EHIP, "admmq_prepare: sync failed");
      break;
    }
    if (hinfo != 0) {
      rc = fail(QZ_ESOLVER, "admmq_prepare: eigensolver did not converge (info " +
                                std::to_string(hinfo) + ")");
      break;
    }
    dim3 grid(static_cast<unsigned>(ceil_div(d, 32)), static_cast<unsigned>(ceil_div(d, 32)));
    export_kernel<<<grid, kThreads, 0, s>>>(A, D, d, V, Lambda);
    if ((rc = check_launch("eig.export")) != QZ_OK) break;
    if (hipStreamSynchronize(s) != hipSuccess) {
      rc = fail(QZ_EHIP, "admmq_prepare: sync failed");
      break;
    }
  } while (false);
  cleanup();
  return rc;
}

}  // namespace qz
