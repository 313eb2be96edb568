// W8A16 skinny GEMM on the matrix cores, 1 <= M <= 16:
//     out[m, n] = alpha * sum_k x[m, k] * dec(W[n, k])
//
// What is computed is the "Matmul2dFp8" page's W8A16 GEMM (bf16 activation,
// float8_e4m3fn weight, float32 accumulation).  At M <= 16 the product is
// still bound by the weight read, but M float32 FMAs per weight byte exceed
// the vector ALU budget, so each 16 x 32 weight slice goes through one
// v_mfma_f32_16x16x32_bf16 with the M activation rows (zero-padded to 16)
// as the other operand.  The E4M3 -> bf16 widening is exact, so the matrix
// core sees exactly the decoded weight.
//
// Work split: a 256-thread block owns 16*G output columns; its four waves
// take interleaved 64-byte K steps, each lane loading one 16-byte chunk per
// row group per step (row l % 16, bytes 16*(l/16) .. +15 of the step), and
// the four partial accumulators are summed through LDS at the end.  The
// same k-slot assignment is used for both operands, so the pairing of
// activation and weight elements does not depend on how the matrix core
// orders the k-slots internally.
#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

template <int G, int U>
__global__ __launch_bounds__(256) void fp8_skinny_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, void* __restrict__ out,
    int out_bf16, int M, int64_t N, int64_t K, float alpha) {
  constexpr int kWaves = 4;
  __shared__ v4f red[kWaves][G][kWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int r16 = lane & 15;   // operand row: m for x, n - n0 - 16g for W
  const int kq = lane >> 4;    // which 16-byte chunk of the 64-byte step
  const int64_t n0 = int64_t(blockIdx.x) * 16 * G;

  const uint8_t* wrow[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    int64_t n = n0 + 16 * g + r16;
    if (n >= N) n = N - 1;  // padding columns re-read the last row; never stored
    wrow[g] = w + n * K;
  }
  const bool xrow_ok = r16 < M;
  const uint16_t* xrow = x + int64_t(xrow_ok ? r16 : 0) * K;

  v4f acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t nsteps = (K + 63) / 64;
  for (int64_t s0 = wid; s0 < nsteps; s0 += int64_t(kWaves) * U) {
    u32x4 wv[U][G];
    u32x4 xv[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kb = (s0 + int64_t(u) * kWaves) * 64 + kq * 16;
      const bool ok = kb < K;  // K % 16 == 0: a chunk is wholly inside or outside
#pragma unroll
      for (int g = 0; g < G; ++g) wv[u][g] = ok ? ld16_stream(wrow[g] + kb) : u32x4{0u, 0u, 0u, 0u};
      const bool xok = ok && xrow_ok;
      xv[u][0] = xok ? ld16(xrow + kb) : u32x4{0u, 0u, 0u, 0u};
      xv[u][1] = xok ? ld16(xrow + kb + 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const v8bf a0 = __builtin_bit_cast(v8bf, xv[u][0]);
      const v8bf a1 = __builtin_bit_cast(v8bf, xv[u][1]);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const v8bf b0 = e4m3x8_to_bf16x8(wv[u][g].x, wv[u][g].y);
        const v8bf b1 = e4m3x8_to_bf16x8(wv[u][g].z, wv[u][g].w);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc[g], 0, 0, 0);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc[g], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int g = 0; g < G; ++g) red[wid][g][lane] = acc[g];
  __syncthreads();

  // Thread (wid, lane) finishes accumulator element v = wid of every lane:
  // D[i][j] with i = m = 4*(lane/16) + wid and j = column n0 + 16g + lane%16.
  const int m = 4 * (lane >> 4) + wid;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) s += red[q][g][lane][wid];
    const int64_t n = n0 + 16 * g + r16;
    if (m < M && n < N) store_out(out, int64_t(m) * N + n, s, alpha, out_bf16);
  }
}

hipError_t launch_fp8_skinny(const uint8_t* w, const uint16_t* x, void* out, int out_bf16,
                             int64_t M, int64_t N, int64_t K, float alpha, int num_cus,
                             hipStream_t s) {
  // Wider column groups per block once there are enough blocks to go round.
  const int64_t blocks16 = (N + 15) / 16;
  if (blocks16 >= int64_t(num_cus) * 16) {
    const int64_t blocks = (N + 63) / 64;
    return launch(fp8_skinny_kernel<4, 2>, dim3(blocks), dim3(256), 0, s, w, x, out, out_bf16,
                  int(M), N, K, alpha);
  }
  return launch(fp8_skinny_kernel<1, 4>, dim3(blocks16), dim3(256), 0, s, w, x, out, out_bf16,
                int(M), N, K, alpha);
}

}  // namespace qlinear
