// qlinear_fp8_gemm_noalloc: the W8A16 matmul of qlinear_fp8_gemm_ws for
// callers that cannot allocate device memory (code under graph capture,
// tight serving loops, hosts that forbid allocation).  Its split-K partial
// sums go to a fixed device array of this file instead of a caller-given
// workspace; the kernels are the ones qlinear_fp8_gemm_ws runs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qlinear.h"

namespace qlinear {
int fp8_gemm_impl(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                  float alpha, int path, void* ws, int64_t ws_bytes, void* stream, const qlinear_epilogue* epilogue);
}

// 8 MiB: the float32 partial planes of every split-K shape of the decode
// workloads (M = 16, N = 4096, K = 14336 takes 2 MiB).  Each device holds its
// own copy from the library's load until the process ends.
static constexpr int64_t kScratchBytes = int64_t(8) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch` (null on failure).  In host code
// the array's name is only a stand-in for the symbol, so the device address
// is looked up once per device, with that device current, and kept.
void* scratch_ptr(int dev) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int qlinear_fp8_gemm_noalloc(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N,
                                        int64_t K, float alpha, const qlinear_epilogue* epilogue, int path,
                                        void* stream) {
  int64_t need = 0;
  if (int st = qlinear_gemm_workspace_size(QLINEAR_WEIGHT_FP8, path, M, N, K, &need)) return st;
  if (need > kScratchBytes) return QLINEAR_ERR_SCRATCH_LIMIT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLINEAR_ERR_DEVICE;
  void* ws = scratch_ptr(dev);
  if (!ws) return QLINEAR_ERR_DEVICE;
  return qlinear::fp8_gemm_impl(w, x, out, out_dtype, M, N, K, alpha, path, ws, kScratchBytes, stream, epilogue);
}
