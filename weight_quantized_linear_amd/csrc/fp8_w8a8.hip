// FP8 W8A8: the static per-tensor E4M3 activation quantiser and the
// fp8 x fp8 -> float32 GEMM for shapes the pipelined LDS kernel does not take.
//
// What is computed: the "fp8_gemv" page's FP8 weight with the activation
// also in float8_e4m3fn.  Its "Scale contract" paragraph notes that the
// checkpoint's per-tensor input_scale cancels only while the activation stays
// bfloat16; with fp8 activations it is the quantisation step:
//     q[m, k] = E4M3(clamp(x[m, k] / input_scale, -448, 448))
// (one IEEE float32 division, round to nearest even), and
//     out[m, n] = alpha * sum_k dec(q[m, k]) * dec(W[n, k]),
// alpha = input_scale * weight_scale, every product exact in float32.
//
// Quantiser: elementwise, eight values (one 16-byte load) per thread; the
// float32 quotient is clamped to the E4M3 range and converted by the hardware
// (v_cvt_pk_fp8_f32, round to nearest even; the GPU tests compare every
// bfloat16 input against the CPU encoder).
#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

namespace {

__device__ __forceinline__ float fp8_quotient(float x, float s) {
  return fminf(fmaxf(x / s, -448.f), 448.f);  // IEEE division; NaN inputs are out of contract
}

// Two floats (within +-448) -> two E4M3 codes in the low 16 bits.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// Fast path: count % 8 == 0, x 16-byte and q 8-byte aligned; thread t
// converts elements 8t .. 8t + 7 of the flattened [M, K] activation.
__global__ __launch_bounds__(256) void fp8_quantize_vec_kernel(const uint16_t* __restrict__ x,
                                                               uint8_t* __restrict__ q, float s,
                                                               int64_t chunks) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks; c += stride) {
    const u32x4 v = ld16(x + c * 8);
    uint32_t lo = 0, hi = 0;
    lo = f32x2_to_e4m3x2(fp8_quotient(bf16lo(v.x), s), fp8_quotient(bf16hi(v.x), s)) |
         (f32x2_to_e4m3x2(fp8_quotient(bf16lo(v.y), s), fp8_quotient(bf16hi(v.y), s)) << 16);
    hi = f32x2_to_e4m3x2(fp8_quotient(bf16lo(v.z), s), fp8_quotient(bf16hi(v.z), s)) |
         (f32x2_to_e4m3x2(fp8_quotient(bf16lo(v.w), s), fp8_quotient(bf16hi(v.w), s)) << 16);
    *reinterpret_cast<u32x2*>(q + c * 8) = u32x2{lo, hi};
  }
}

// Any size and alignment: one element per thread.
__global__ __launch_bounds__(256) void fp8_quantize_any_kernel(const uint16_t* __restrict__ x,
                                                               uint8_t* __restrict__ q, float s,
                                                               int64_t count) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride)
    q[i] = uint8_t(f32x2_to_e4m3x2(fp8_quotient(bf16_to_f32(x[i]), s), 0.f) & 0xFFu);
}

// Fallback GEMM (any K, any alignment): one output per thread, float32 FMA
// over K (each product of two E4M3 values is exact in float32).  A 256-thread
// block covers 16 rows x 16 columns; slow, for shapes off the fast path only.
__global__ __launch_bounds__(256) void fp8_w8a8_any_kernel(const uint8_t* __restrict__ xq,
                                                           const uint8_t* __restrict__ w,
                                                           void* __restrict__ out, int out_bf16, int64_t M,
                                                           int64_t N, int64_t K, float alpha) {
  const int64_t m = int64_t(blockIdx.y) * 16 + threadIdx.x / 16;
  const int64_t n = int64_t(blockIdx.x) * 16 + threadIdx.x % 16;
  if (m >= M || n >= N) return;
  const uint8_t* xr = xq + m * K;
  const uint8_t* wr = w + n * K;
  float acc = 0.f;
  for (int64_t k = 0; k < K; ++k) acc = fmaf(e4m3_to_f32(xr[k]), e4m3_to_f32(wr[k]), acc);
  store_out(out, m * N + n, acc, alpha, out_bf16);
}

}  // namespace

hipError_t launch_fp8_quantize_act(const uint16_t* x, uint8_t* q, float input_scale, int64_t M, int64_t K,
                                   int num_cus, hipStream_t s) {
  const int64_t count = M * K;
  const bool vec = count % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(q) % 8 == 0;
  const int64_t items = vec ? count / 8 : count;
  int64_t blocks = (items + 255) / 256;
  const int64_t cap = int64_t(num_cus) * 16;
  if (blocks > cap) blocks = cap;
  if (vec)
    return launch(fp8_quantize_vec_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, x, q, input_scale, items);
  return launch(fp8_quantize_any_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, x, q, input_scale, items);
}

hipError_t launch_fp8_w8a8_gemm(const uint8_t* xq, const uint8_t* w, void* out, int out_bf16, int64_t M, int64_t N,
                                int64_t K, float alpha, int num_cus, hipStream_t s) {
  if (int8_lds_supported(xq, w, M, N, K))  // same operand layout and limits as the int8 kernel
    return launch_fp8_w8a8_lds(xq, w, out, out_bf16, M, N, K, alpha, num_cus, s);
  const dim3 grid(unsigned((N + 15) / 16), unsigned((M + 15) / 16));
  return launch(fp8_w8a8_any_kernel, grid, dim3(256), 0, s, xq, w, out, out_bf16, M, N, K, alpha);
}

}  // namespace qlinear
