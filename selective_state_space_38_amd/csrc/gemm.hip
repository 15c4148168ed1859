// Plain row-major GEMMs for the Mamba block's projections, through rocBLAS
// (the projections are ordinary dense matrix products; rocBLAS runs them on
// the MFMA units).  One rocBLAS handle per host thread and device, created on
// first use and destroyed when the thread exits, so concurrent callers on
// different threads never share a handle's stream setting.

#include <rocblas/rocblas.h>

#include <unordered_map>

#include "ssm_internal.h"

namespace ssm {

namespace {

struct HandleCache {
  std::unordered_map<int, rocblas_handle> by_device;
  ~HandleCache() {
    for (auto& kv : by_device) rocblas_destroy_handle(kv.second);
  }
};

rocblas_handle handle_for_current_device() {
  thread_local HandleCache cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  auto it = cache.by_device.find(dev);
  if (it != cache.by_device.end()) return it->second;
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
  cache.by_device.emplace(dev, h);
  return h;
}

}  // namespace

// C[M][N] = A[M][K] * W[K][N], all row-major with leading dimensions lda,
// ldw, ldc (elements); dtype 0 = float32, 1 = bfloat16 storage, float32
// accumulation.  In rocBLAS's column-major terms this is C^T = W^T A^T.
hipError_t gemm_rowmajor(int dtype, int64_t M, int64_t N, int64_t K, const void* A,
                         int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc,
                         hipStream_t stream) {
  rocblas_handle h = handle_for_current_device();
  if (!h) return hipErrorUnknown;
  if (rocblas_set_stream(h, stream) != rocblas_status_success) return hipErrorUnknown;
  const rocblas_datatype t = dtype == 0 ? rocblas_datatype_f32_r : rocblas_datatype_bf16_r;
  const float alpha = 1.0f, beta = 0.0f;
  const rocblas_status st = rocblas_gemm_ex(
      h, rocblas_operation_none, rocblas_operation_none, static_cast<rocblas_int>(N),
      static_cast<rocblas_int>(M), static_cast<rocblas_int>(K), &alpha, W, t,
      static_cast<rocblas_int>(ldw), A, t, static_cast<rocblas_int>(lda), &beta, C, t,
      static_cast<rocblas_int>(ldc), C, t, static_cast<rocblas_int>(ldc),
      rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? hipSuccess : hipErrorUnknown;
}

}  // namespace ssm
