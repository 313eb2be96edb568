// W4A16 NVFP4 on the vector ALU (1 <= M <= 4) and NVFP4 dequantisation.
//
// Format ("fp4_matmul" page, summary): the weight stays packed, uint8
// [N, K/2] with two E2M1 codes per byte (even k in the low nibble), plus one
// float8_e4m3fn block scale per 16 consecutive k of a row, [N, K/16].  The
// dequantised weight is D[n, k] = e2m1(code) * e4m3(scale[n, k/16]); alpha is
// the per-tensor global scale (weight_scale_2, "fp8_gemv" page "Scale
// contract").
//
// The GEMV mirrors the FP8 one: each 64-lane wave owns ROWS weight rows;
// lane l takes the 16-byte packed chunks c = l, l + 64, ... (32 weights and
// two block scales each).  Pairs of nibbles are widened exactly to bfloat16
// (conversion scale 1) and multiplied by the bfloat16 activation pairs with
// v_dot2_f32_bf16 into a float32 partial sum per 16-value block, which is
// then scaled by that block's E4M3 scale and added to the row's float32
// accumulator: one conversion and M/2 dot products per weight pair instead
// of a conversion, two scale products and M fused multiply-adds per pair.
// The block scale distributes over the block's sum, so only the rounding
// order differs from scaling every weight.
#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

namespace {

template <int M, int ROWS>
__global__ __launch_bounds__(256) void nvfp4_gemv_wide_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ x, void* __restrict__ out, int out_bf16, int64_t N, int64_t K,
    float alpha, Epilogue epi) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t row0 = wave * ROWS;
  if (row0 >= N) return;
  const int64_t row_bytes = K >> 1, row_scales = K >> 4;
  const int64_t nchunks = K >> 5;  // 32 weights per 16-byte chunk

  const uint8_t* prow[ROWS];
  const uint16_t* srow[ROWS];  // two scales per chunk -> one 16-bit load
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int64_t row = row0 + r < N ? row0 + r : N - 1;
    prow[r] = packed + row * row_bytes;
    srow[r] = reinterpret_cast<const uint16_t*>(scales + row * row_scales);
  }
  float acc[M][ROWS];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[m][r] = 0.f;

  constexpr int U = 2;
  for (int64_t c0 = 0; c0 < nchunks; c0 += int64_t(kWave) * U) {
    u32x4 wv[U][ROWS];
    uint32_t sv[U][ROWS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + int64_t(u) * kWave + lane;
      const bool ok = c < nchunks;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        wv[u][r] = ok ? ld16_stream(prow[r] + c * 16) : u32x4{0u, 0u, 0u, 0u};
        sv[u][r] = ok ? uint32_t(srow[r][c]) : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + int64_t(u) * kWave + lane;
      const bool ok = c < nchunks;
      // Activation k = 32 c .. 32 c + 31 as bfloat16 pairs: xv[m][q] holds k = 32 c + 8 q .. + 7.
      u32x4 xv[M][4];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[m][q] = ok ? ld16(x + m * K + c * 32 + 8 * q) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {  // dwords 2 blk, 2 blk + 1 = weights 16 blk .. 16 blk + 15
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          float part[M];
#pragma unroll
          for (int m = 0; m < M; ++m) part[m] = 0.f;
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            v2bf wp[4];  // wp[j] = weights 16 blk + 8 d + 2 j, + 1
            e2m1x8_to_bf16x8(wv[u][r][2 * blk + d], wp);
#pragma unroll
            for (int m = 0; m < M; ++m) {
              const u32x4& xa = xv[m][2 * blk + d];
              part[m] = __builtin_amdgcn_fdot2_f32_bf16(wp[0], as_bf16x2(xa.x), part[m], false);
              part[m] = __builtin_amdgcn_fdot2_f32_bf16(wp[1], as_bf16x2(xa.y), part[m], false);
              part[m] = __builtin_amdgcn_fdot2_f32_bf16(wp[2], as_bf16x2(xa.z), part[m], false);
              part[m] = __builtin_amdgcn_fdot2_f32_bf16(wp[3], as_bf16x2(xa.w), part[m], false);
            }
          }
          const float sb = e4m3_to_f32((sv[u][r] >> (8 * blk)) & 0xFFu);
#pragma unroll
          for (int m = 0; m < M; ++m) acc[m][r] = fmaf(sb, part[m], acc[m][r]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float t = wave_sum(acc[m][r]);
      if (lane == 0 && row0 + r < N) store_epi(out, m, row0 + r, N, t, alpha, out_bf16, epi);
    }
}

// One weight at (n, k), decoded to float (exact).
__device__ __forceinline__ float nvfp4_at(const uint8_t* packed, const uint8_t* scales, int64_t n,
                                          int64_t K, int64_t k) {
  const uint32_t byte = packed[n * (K >> 1) + (k >> 1)];
  const float s = e4m3_to_f32(scales[n * (K >> 4) + (k >> 4)]);
  float lo, hi;
  e2m1x2_scaled_f32<0>(byte, s, lo, hi);
  return (k & 1) ? hi : lo;
}

// Any alignment, K % 16 == 0: lane l takes k = l, l + 64, ...
template <int M>
__global__ __launch_bounds__(256) void nvfp4_gemv_any_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ x, void* __restrict__ out, int out_bf16, int64_t N, int64_t K,
    float alpha, Epilogue epi) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= N) return;
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;
  for (int64_t k = lane; k < K; k += kWave) {
    const float wv = nvfp4_at(packed, scales, row, K, k);
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = fmaf(bf16_to_f32(x[m * K + k]), wv, acc[m]);
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float t = wave_sum(acc[m]);
    if (lane == 0) store_epi(out, m, row, N, t, alpha, out_bf16, epi);
  }
}

// Dense dequantisation: bfloat16 output through the decoder of the
// matrix-core GEMM, float32 output through the decoder of the GEMV.
__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ scales,
                                                            void* __restrict__ out, int out_bf16,
                                                            int64_t N, int64_t K) {
  const int64_t pairs = N * (K >> 1);
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t p = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; p < pairs; p += stride) {
    const int64_t n = p / (K >> 1);
    const int64_t k = 2 * (p - n * (K >> 1));
    const uint32_t byte = packed[p];
    const float s = e4m3_to_f32(scales[n * (K >> 4) + (k >> 4)]);
    if (out_bf16) {
      const uint32_t v = e2m1x2_to_bf16x2<0>(byte, s);
      uint16_t* o = reinterpret_cast<uint16_t*>(out) + n * K + k;
      o[0] = uint16_t(v);
      o[1] = uint16_t(v >> 16);
    } else {
      float lo, hi;
      e2m1x2_scaled_f32<0>(byte, s, lo, hi);
      float* o = reinterpret_cast<float*>(out) + n * K + k;
      o[0] = lo;
      o[1] = hi;
    }
  }
}

template <int M>
hipError_t gemv_m(bool wide, const uint8_t* p, const uint8_t* sc, const uint16_t* x, void* out, int bf16,
                  int64_t N, int64_t K, float alpha, int num_cus, const Epilogue& epi, hipStream_t s) {
  if (!wide) {
    const int64_t blocks = (N + 3) / 4;
    return launch(nvfp4_gemv_any_kernel<M>, dim3(blocks), dim3(256), 0, s, p, sc, x, out, bf16, N, K, alpha, epi);
  }
  const int64_t target_waves = int64_t(num_cus) * 8;
  if (N >= target_waves * 4)
    return launch(nvfp4_gemv_wide_kernel<M, 4>, dim3((N + 15) / 16), dim3(256), 0, s, p, sc, x, out, bf16, N,
                  K, alpha, epi);
  if (N >= target_waves * 2)
    return launch(nvfp4_gemv_wide_kernel<M, 2>, dim3((N + 7) / 8), dim3(256), 0, s, p, sc, x, out, bf16, N, K,
                  alpha, epi);
  return launch(nvfp4_gemv_wide_kernel<M, 1>, dim3((N + 3) / 4), dim3(256), 0, s, p, sc, x, out, bf16, N, K,
                alpha, epi);
}

}  // namespace

hipError_t launch_nvfp4_gemv(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* out,
                             int out_bf16, int64_t M, int64_t N, int64_t K, float alpha, int num_cus,
                             hipStream_t s, const Epilogue& epi) {
  const bool wide = (K % 32 == 0) && (reinterpret_cast<uintptr_t>(packed) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(scales) % 2 == 0) &&
                    (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  switch (M) {
    case 1: return gemv_m<1>(wide, packed, scales, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 2: return gemv_m<2>(wide, packed, scales, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 3: return gemv_m<3>(wide, packed, scales, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 4: return gemv_m<4>(wide, packed, scales, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_nvfp4_dequant(const uint8_t* packed, const uint8_t* scales, void* out, int out_bf16,
                                int64_t N, int64_t K, hipStream_t s) {
  const int64_t pairs = N * (K >> 1);
  int64_t blocks = (pairs + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return launch(nvfp4_dequant_kernel, dim3(blocks), dim3(256), 0, s, packed, scales, out, out_bf16, N, K);
}

}  // namespace qlinear
