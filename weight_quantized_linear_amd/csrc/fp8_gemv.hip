// W8A16 GEMV on the vector ALU: out[m, n] = alpha * sum_k x[m, k] * dec(W[n, k])
// for 1 <= M <= 4.
//
// What is computed follows the "fp8_gemv" documentation page (summary,
// "Structure", "Scale contract"): at M = 1 there is one activation row, so
// the product is a matrix-vector product with nothing for a matrix core to
// do; the work is reading the 1-byte weights, widening them exactly and
// accumulating in float32.  The page's kernel gives one 32-lane warp to each
// output; here each 64-lane wave owns ROWS output rows at once and every lane
// issues ROWS x U independent 16-byte weight loads before it consumes any:
// the kernel is bound by HBM bandwidth, and on MI355X it is the burst of
// whole contiguous rows per wave that keeps it near the bandwidth roof (two
// rows per wave measured best on the 128256 x 4096 weight).
//
// Arithmetic: pairs of E4M3 bytes are widened to pairs of bfloat16 with the
// hardware conversion (exact: every E4M3 value fits bfloat16) and multiplied
// by the bfloat16 activation pairs with v_dot2c_f32_bf16, which accumulates
// in float32.  Every product of two bfloat16 values is exact in float32, so
// this computes the same products as widening both operands to float32 and
// using FMAs, at half the vector-ALU instructions per weight.
#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

// Wide path: K % 16 == 0 and 16-byte aligned bases.  Lane `l` handles the
// 16-byte chunks c = l, l + 64, l + 128, ... of each row; U chunks per lane
// are loaded before any is used.
template <int M, int ROWS, int U>
__global__ __launch_bounds__(256) void fp8_gemv_wide_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, void* __restrict__ out,
    int out_bf16, int64_t N, int64_t K, float alpha, Epilogue epi) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t row0 = wave * ROWS;
  if (row0 >= N) return;  // uniform per wave

  const int64_t nchunks = K >> 4;
  const uint8_t* wrow[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int64_t row = row0 + r < N ? row0 + r : N - 1;  // tail rows re-read the last row, never stored
    wrow[r] = w + row * K;
  }

  float acc[M][ROWS];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[m][r] = 0.f;

  for (int64_t c0 = 0; c0 < nchunks; c0 += int64_t(kWave) * U) {
    u32x4 wv[U][ROWS];
    u32x4 xv[U][M][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + int64_t(u) * kWave + lane;
      const bool ok = c < nchunks;
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
        wv[u][r] = ok ? ld16_stream(wrow[r] + c * 16) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint16_t* xp = x + m * K + c * 16;
        xv[u][m][0] = ok ? ld16(xp) : u32x4{0u, 0u, 0u, 0u};
        xv[u][m][1] = ok ? ld16(xp + 8) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {  // dword d of the chunk = elements 4d .. 4d+3
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const v2bf w01 = __builtin_bit_cast(v2bf, e4m3x2_to_bf16x2<false>(wv[u][r][d]));
          const v2bf w23 = __builtin_bit_cast(v2bf, e4m3x2_to_bf16x2<true>(wv[u][r][d]));
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const u32x4& xa = xv[u][m][d >> 1];
            const v2bf x01 = __builtin_bit_cast(v2bf, (d & 1) ? xa.z : xa.x);
            const v2bf x23 = __builtin_bit_cast(v2bf, (d & 1) ? xa.w : xa.y);
            acc[m][r] = __builtin_amdgcn_fdot2_f32_bf16(w01, x01, acc[m][r], false);
            acc[m][r] = __builtin_amdgcn_fdot2_f32_bf16(w23, x23, acc[m][r], false);
          }
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float s = wave_sum(acc[m][r]);
      if (lane == 0 && row0 + r < N) store_epi(out, m, row0 + r, N, s, alpha, out_bf16, epi);
    }
}

// Any K, any alignment: lane `l` reads the bytes k = l, l + 64, ... of each
// row (coalesced one-byte loads), four at a time.
template <int M, int ROWS>
__global__ __launch_bounds__(256) void fp8_gemv_any_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, void* __restrict__ out,
    int out_bf16, int64_t N, int64_t K, float alpha, Epilogue epi) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t row0 = wave * ROWS;
  if (row0 >= N) return;

  const uint8_t* wrow[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) wrow[r] = w + (row0 + r < N ? row0 + r : N - 1) * K;

  float acc[M][ROWS];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[m][r] = 0.f;

  constexpr int U = 4;
  for (int64_t k0 = 0; k0 < K; k0 += int64_t(kWave) * U) {
    uint32_t wb[U][ROWS];
    float xf[U][M];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + int64_t(u) * kWave + lane;
      const bool ok = k < K;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) wb[u][r] = ok ? uint32_t(wrow[r][k]) : 0u;
#pragma unroll
      for (int m = 0; m < M; ++m) xf[u][m] = ok ? bf16_to_f32(x[m * K + k]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const float wf = e4m3_to_f32(wb[u][r]);
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m][r] = fmaf(xf[u][m], wf, acc[m][r]);
      }
  }

#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float s = wave_sum(acc[m][r]);
      if (lane == 0 && row0 + r < N) store_epi(out, m, row0 + r, N, s, alpha, out_bf16, epi);
    }
}

namespace {

template <int M, int ROWS>
hipError_t launch_rows(bool wide, const uint8_t* w, const uint16_t* x, void* out, int out_bf16,
                       int64_t N, int64_t K, float alpha, const Epilogue& epi, hipStream_t s) {
  constexpr int kThreads = 256;
  constexpr int kRowsPerBlock = ROWS * (kThreads / kWave);
  const int64_t blocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  if (wide) {
    // U chunks of 1 KiB per row are in flight per lane-group; short rows take
    // U = 2 so that no loads are padding, longer rows U = 4 (M = 1) or 2.
    const int64_t per_lane = ((K >> 4) + kWave - 1) / kWave;
    if (M > 1 || per_lane <= 2)
      return launch(fp8_gemv_wide_kernel<M, ROWS, 2>, dim3(blocks), dim3(kThreads), 0, s, w, x, out,
                    out_bf16, N, K, alpha, epi);
    return launch(fp8_gemv_wide_kernel<M, ROWS, 4>, dim3(blocks), dim3(kThreads), 0, s, w, x, out,
                  out_bf16, N, K, alpha, epi);
  }
  return launch(fp8_gemv_any_kernel<M, ROWS>, dim3(blocks), dim3(kThreads), 0, s, w, x, out,
                out_bf16, N, K, alpha, epi);
}

template <int M>
hipError_t launch_m(bool wide, const uint8_t* w, const uint16_t* x, void* out, int out_bf16,
                    int64_t N, int64_t K, float alpha, int num_cus, const Epilogue& epi, hipStream_t s) {
  // Two rows per wave once that still gives every SIMD several waves.
  if (N >= int64_t(num_cus) * 16) return launch_rows<M, 2>(wide, w, x, out, out_bf16, N, K, alpha, epi, s);
  return launch_rows<M, 1>(wide, w, x, out, out_bf16, N, K, alpha, epi, s);
}

}  // namespace

hipError_t launch_fp8_gemv(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M,
                           int64_t N, int64_t K, float alpha, int num_cus, hipStream_t s, const Epilogue& epi) {
  const bool wide = (K % 16 == 0) && (reinterpret_cast<uintptr_t>(w) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  switch (M) {
    case 1: return launch_m<1>(wide, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 2: return launch_m<2>(wide, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 3: return launch_m<3>(wide, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 4: return launch_m<4>(wide, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlinear
