// FP8 weight materialisation ("fp8_gemv" page, enqueue_fp8_materialize /
// fp8_materialize_kernel): out[i] = dec_e4m3(w[i]) over the dense [N, K]
// weight.  The float32 output goes through the decoder of the vector-ALU
// GEMV and the bfloat16 output through the decoder of the matrix-core
// kernels, so an exhaustive 256-code check of this call checks both.
#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

__global__ __launch_bounds__(256) void fp8_materialize_kernel(const uint8_t* __restrict__ w,
                                                              void* __restrict__ out, int out_bf16,
                                                              int64_t count) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t * 4 < count; t += stride) {
    const int64_t i0 = t * 4;
    uint32_t packed = 0;
    const int n = count - i0 < 4 ? int(count - i0) : 4;
    for (int e = 0; e < n; ++e) packed |= uint32_t(w[i0 + e]) << (8 * e);
    if (out_bf16) {
      const uint32_t lo = e4m3x2_to_bf16x2<false>(packed);
      const uint32_t hi = e4m3x2_to_bf16x2<true>(packed);
      const uint16_t v[4] = {uint16_t(lo), uint16_t(lo >> 16), uint16_t(hi), uint16_t(hi >> 16)};
      uint16_t* o = reinterpret_cast<uint16_t*>(out) + i0;
      for (int e = 0; e < n; ++e) o[e] = v[e];
    } else {
      float v[4];
      e4m3x4_to_f32(packed, v);
      float* o = reinterpret_cast<float*>(out) + i0;
      for (int e = 0; e < n; ++e) o[e] = v[e];
    }
  }
}

hipError_t launch_fp8_materialize(const uint8_t* w, void* out, int out_bf16, int64_t count,
                                  hipStream_t s) {
  const int64_t groups = (count + 3) / 4;
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return launch(fp8_materialize_kernel, dim3(blocks), dim3(256), 0, s, w, out, out_bf16, count);
}

}  // namespace qlinear
