// Host-side launch helper and the internal entry points that the C ABI
// (qlinear.cpp) dispatches to.  Each launcher only enqueues; it returns the
// HIP error of the launch itself.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "epilogue.hpp"

namespace qlinear {

// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per device: the attribute belongs to the device the call is made on, so a
// process that launches on several GPUs sets it on each.  `done` keeps one
// bit per device id below 64 (higher ids set it on every call); concurrent
// first calls from several host threads may both set it, which is harmless.
inline hipError_t raise_lds_limit(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  if (hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); e != hipSuccess)
    return e;
  done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

template <typename T> struct same_type { using type = T; };

// Launch through hipLaunchKernel so the launch status comes back directly
// (no reliance on the thread's sticky last-error state).  Arguments are
// converted to the kernel's own parameter types first.
template <typename... Params>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                  typename same_type<Params>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem, s);
}

// fp8_gemv.hip
hipError_t launch_fp8_gemv(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M,
                           int64_t N, int64_t K, float alpha, int num_cus, hipStream_t s, const Epilogue& epi = Epilogue{});

// fp8_skinny.hip
// True when the activation-resident matrix-core kernel serves (M, N, K)
// (M <= 8, K % 256 == 0, the zero-padded activation fits in LDS).
bool fp8_skinny_xlds_supported(int64_t M, int64_t N, int64_t K);
// True where the streaming matrix-core kernel is the measured best skinny
// kernel for (M, N, K), given that it supports the shape.
bool fp8_skinny_stream_wins(int64_t M, int64_t N, int64_t K);
hipError_t launch_fp8_skinny(const uint8_t* w, const uint16_t* x, void* out, int out_bf16,
                             int64_t M, int64_t N, int64_t K, float alpha, int num_cus,
                             hipStream_t s, const Epilogue& epi = Epilogue{});

// Split-K skinny GEMM (M <= 16, K % 64 == 0, aligned, workspace present):
// the streaming kernel's split-K form where K is made of 2048-value slices
// and the workspace holds its planes, else the split-K skinny kernel;
// hipErrorInvalidValue when the shape does not suit it.  The second kernel
// (gemm_lds.hip) adds the float32 partial planes [splits, M, N] in order,
// then applies alpha and the epilogue.
hipError_t launch_fp8_skinny_splitk(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M,
                                   int64_t N, int64_t K, float alpha, int num_cus, float* ws, size_t ws_bytes,
                                   hipStream_t s, const Epilogue& epi = Epilogue{});
hipError_t launch_splitk_reduce(const float* part, void* out, int out_bf16, int64_t M, int64_t N, int splits,
                                float alpha, hipStream_t s, const Epilogue& epi = Epilogue{});
// Streaming skinny kernel (M <= 16, K in {1024, 2048, 3072, 4096}, 16-byte
// aligned weight and activation): weight tiles of 16 rows DMA'd whole into
// an LDS ring; hipErrorInvalidValue when the shape does not suit it.
bool fp8_skinny_stream_supported(const void* w, const void* x, int64_t M, int64_t N, int64_t K);
hipError_t launch_fp8_skinny_stream(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M,
                                    int64_t N, int64_t K, float alpha, int num_cus, hipStream_t s,
                                    const Epilogue& epi = Epilogue{});
// Workspace bytes a split-K skinny call takes for (M, N, K): room for the
// planes of either split-K kernel (0: split-K does not apply).
size_t fp8_skinny_splitk_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus);

// gemm_bf16.hip (dispatches to gemm_lds.hip when K % 64 == 0 and operands are aligned)
hipError_t launch_fp8_tiled(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M,
                            int64_t N, int64_t K, float alpha, int num_cus, float* ws, size_t ws_bytes,
                            hipStream_t s, const Epilogue& epi = Epilogue{});
hipError_t launch_nvfp4_tiled(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* out,
                              int out_bf16, int64_t M, int64_t N, int64_t K, float alpha, int num_cus, float* ws,
                              size_t ws_bytes, hipStream_t s, const Epilogue& epi = Epilogue{});

// gemm_lds.hip
bool gemm_lds_supported(const void* x, const void* w, const void* scales, int64_t M, int64_t N, int64_t K);
// ws / ws_bytes: the caller's float32 workspace for split-K partial sums (null: whole-K tiles only).
hipError_t launch_fp8_gemm_lds(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                               int64_t K, float alpha, int num_cus, float* ws, size_t ws_bytes, hipStream_t s, const Epilogue& epi = Epilogue{});
// Workspace bytes with which the LDS GEMMs take their split-K kernels (0: whole-K tiles).
size_t fp8_gemm_lds_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus);
size_t nvfp4_gemm_lds_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus);
size_t bf16_gemm_lds_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus);
bool int8_lds_supported(const void* a, const void* b, int64_t M, int64_t N, int64_t K);
hipError_t launch_int8_gemm_lds(const int8_t* a, const int8_t* b, const float* sa, const float* sb,
                                const uint16_t* bias, void* out, int out_mode, int64_t M, int64_t N, int64_t K,
                                int num_cus, hipStream_t s);
hipError_t launch_nvfp4_gemm_lds(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* out,
                                 int out_bf16, int64_t M, int64_t N, int64_t K, float alpha, int num_cus, float* ws,
                                 size_t ws_bytes, hipStream_t s, const Epilogue& epi = Epilogue{});
bool grouped_lds_supported(const void* x, const void* w, int64_t G, int64_t T, int64_t N, int64_t K);
hipError_t launch_fp8_grouped_lds(const uint8_t* w, const uint16_t* x, const uint32_t* a_offsets,
                                  const int32_t* expert_ids, void* out, int out_bf16, int64_t G, int64_t E, int64_t T,
                                  int64_t N, int64_t K, int num_cus, hipStream_t s, const float* expert_scale = nullptr);
hipError_t launch_fp8_grouped(const uint8_t* w, const uint16_t* x, const uint32_t* a_offsets,
                              const int32_t* expert_ids, void* out, int out_bf16, int64_t G,
                              int64_t max_tokens, int64_t E, int64_t T, int64_t N, int64_t K,
                              int num_cus, hipStream_t s, const float* expert_scale = nullptr);
bool nvfp4_grouped_lds_supported(const void* x, const void* packed, const void* scales, int64_t G, int64_t T,
                                 int64_t N, int64_t K);
hipError_t launch_nvfp4_grouped_lds(const uint8_t* packed, const uint8_t* scales, const uint16_t* x,
                                    const uint32_t* a_offsets, const int32_t* expert_ids, void* out, int out_bf16,
                                    int64_t G, int64_t E, int64_t T, int64_t N, int64_t K, int num_cus,
                                    hipStream_t s, const float* expert_scale = nullptr);
// Grouped NVFP4 (expert stacks [E, N, K/2] and [E, N, K/16], K % 16 == 0).
hipError_t launch_nvfp4_grouped(const uint8_t* packed, const uint8_t* scales, const uint16_t* x,
                                const uint32_t* a_offsets, const int32_t* expert_ids, void* out, int out_bf16,
                                int64_t G, int64_t max_tokens, int64_t E, int64_t T, int64_t N, int64_t K,
                                int num_cus, hipStream_t s, const float* expert_scale = nullptr);

// fp8_w8a8.hip (FP8 activations: static per-tensor quantiser, fp8 x fp8 GEMM)
hipError_t launch_fp8_quantize_act(const uint16_t* x, uint8_t* q, float input_scale, int64_t M, int64_t K,
                                   int num_cus, hipStream_t s);
hipError_t launch_fp8_w8a8_gemm(const uint8_t* xq, const uint8_t* w, void* out, int out_bf16, int64_t M, int64_t N,
                                int64_t K, float alpha, int num_cus, hipStream_t s);
// gemm_lds.hip: the pipelined fp8 x fp8 kernel (K % 64 == 0, aligned, int8_lds_supported).
hipError_t launch_fp8_w8a8_lds(const uint8_t* xq, const uint8_t* w, void* out, int out_bf16, int64_t M, int64_t N,
                               int64_t K, float alpha, int num_cus, hipStream_t s);

// nvfp4.hip
// Dense bf16 control (bf16_dense.hip, gemm_lds.hip, gemm_bf16.hip).
bool bf16_wide(const void* w, const void* x, int64_t K);
hipError_t launch_bf16_gemv(const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                            int64_t K, float alpha, int num_cus, hipStream_t s, const Epilogue& epi = Epilogue{});
hipError_t launch_bf16_skinny(const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                              int64_t K, float alpha, int num_cus, hipStream_t s, const Epilogue& epi = Epilogue{});
bool bf16_lds_supported(const void* x, const void* w, int64_t M, int64_t N, int64_t K);
hipError_t launch_bf16_gemm_lds(const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                                int64_t K, float alpha, int num_cus, float* ws, size_t ws_bytes, hipStream_t s, const Epilogue& epi = Epilogue{});
hipError_t launch_bf16_tiled(const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                             int64_t K, float alpha, int num_cus, float* ws, size_t ws_bytes, hipStream_t s, const Epilogue& epi = Epilogue{});

hipError_t launch_nvfp4_gemv(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* out,
                             int out_bf16, int64_t M, int64_t N, int64_t K, float alpha, int num_cus,
                             hipStream_t s, const Epilogue& epi = Epilogue{});
hipError_t launch_nvfp4_dequant(const uint8_t* packed, const uint8_t* scales, void* out, int out_bf16,
                                int64_t N, int64_t K, hipStream_t s);

// int8.hip
hipError_t launch_int8_quantize(const uint16_t* x, int8_t* q, float* a_scale, int64_t M, int64_t K,
                                hipStream_t s);
bool int8_grouped_lds_supported(const void* a, const void* b, int64_t G, int64_t T, int64_t N, int64_t K);
hipError_t launch_int8_grouped_lds(const int8_t* a, const int8_t* b, const float* sa, const float* sb,
                                   const uint16_t* bias, const uint32_t* a_offsets, const int32_t* expert_ids,
                                   void* out, int out_mode, int64_t G, int64_t E, int64_t T, int64_t N, int64_t K,
                                   int num_cus, hipStream_t s);
hipError_t launch_int8_grouped(const int8_t* a, const int8_t* b, const float* a_scale, const float* b_scale,
                               const uint16_t* bias, const uint32_t* a_offsets, const int32_t* expert_ids, void* out,
                               int out_mode, int64_t G, int64_t max_tokens, int64_t E, int64_t T, int64_t N, int64_t K,
                               int num_cus, hipStream_t s);
hipError_t launch_int8_gemm(const int8_t* a, const int8_t* b, const float* a_scale, const float* b_scale,
                            const uint16_t* bias, void* out, int out_mode, int64_t M, int64_t N, int64_t K,
                            int num_cus, hipStream_t s);

// materialize.hip
hipError_t launch_fp8_materialize(const uint8_t* w, void* out, int out_bf16, int64_t count,
                                  hipStream_t s);

}  // namespace qlinear
