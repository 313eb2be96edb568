// Dense bf16 control: out[m, n] = alpha * sum_k x[m, k] * W[n, k] with a
// bfloat16 weight, for 1 <= M <= 16 (M > 16 runs the LDS-tiled GEMM of
// gemm_lds.hip with an undecoded bf16 weight operand).
//
// What is computed: the dense bf16 weight path that the quantized kernels are
// measured against -- the fp8_gemv page ("WHY it wins at decode") attributes
// the whole W8A16 decode gain to reading 1 byte per weight instead of 2, and
// the Matmul2dFp8 page (summary) describes its tiled kernel as the dense bf16
// GEMM with only the weight type changed.  These kernels are the same
// designs as the FP8 GEMV and skinny kernels with the weight read as stored:
// no decode, twice the bytes per weight.
//
// * bf16_gemv_wide_kernel (M <= 4, K % 8 == 0, aligned): a wave owns ROWS
//   weight rows; every lane issues ROWS x U independent 16-byte loads (eight
//   weights each) before using any, and multiplies bf16 pairs with
//   v_dot2c_f32_bf16 into float32 (each product of two bf16 values is exact
//   in float32).
// * bf16_gemv_any_kernel: any K and alignment, one element per lane step.
// * bf16_skinny_kernel (5 <= M <= 16, K % 8 == 0, aligned): v_mfma_f32_16x16x32_bf16
//   with the activation rows (zero-padded to 16) as one operand and 16
//   weight rows per group as the other; a lane's 16-byte load is exactly one
//   operand fragment.  NWV waves take interleaved K steps and add their
//   partial accumulators through LDS.
#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

namespace {

template <int M, int ROWS, int U>
__global__ __launch_bounds__(256) void bf16_gemv_wide_kernel(const uint16_t* __restrict__ w,
                                                             const uint16_t* __restrict__ x, void* __restrict__ out,
                                                             int out_bf16, int64_t N, int64_t K, float alpha, Epilogue epi) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t row0 = wave * ROWS;
  if (row0 >= N) return;  // uniform per wave

  const int64_t nchunks = K >> 3;  // 16-byte chunks of 8 values per row
  const uint16_t* wrow[ROWS];
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
    u32x4 xv[U][M];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + int64_t(u) * kWave + lane;
      const bool ok = c < nchunks;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) wv[u][r] = ok ? ld16_stream(wrow[r] + c * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int m = 0; m < M; ++m) xv[u][m] = ok ? ld16(x + m * K + c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int d = 0; d < 4; ++d)  // dword d of the chunk = elements 2d, 2d + 1
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
          for (int m = 0; m < M; ++m)
            acc[m][r] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wv[u][r][d]), as_bf16x2(xv[u][m][d]), acc[m][r],
                                                        false);
  }

#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float s = wave_sum(acc[m][r]);
      if (lane == 0 && row0 + r < N) store_epi(out, m, row0 + r, N, s, alpha, out_bf16, epi);
    }
}

template <int M, int ROWS>
__global__ __launch_bounds__(256) void bf16_gemv_any_kernel(const uint16_t* __restrict__ w,
                                                            const uint16_t* __restrict__ x, void* __restrict__ out,
                                                            int out_bf16, int64_t N, int64_t K, float alpha, Epilogue epi) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t row0 = wave * ROWS;
  if (row0 >= N) return;

  const uint16_t* wrow[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) wrow[r] = w + (row0 + r < N ? row0 + r : N - 1) * K;

  float acc[M][ROWS];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[m][r] = 0.f;

  constexpr int U = 4;
  for (int64_t k0 = 0; k0 < K; k0 += int64_t(kWave) * U) {
    float wf[U][ROWS], xf[U][M];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + int64_t(u) * kWave + lane;
      const bool ok = k < K;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) wf[u][r] = ok ? bf16_to_f32(wrow[r][k]) : 0.f;
#pragma unroll
      for (int m = 0; m < M; ++m) xf[u][m] = ok ? bf16_to_f32(x[m * K + k]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m][r] = fmaf(xf[u][m], wf[u][r], acc[m][r]);
  }

#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float s = wave_sum(acc[m][r]);
      if (lane == 0 && row0 + r < N) store_epi(out, m, row0 + r, N, s, alpha, out_bf16, epi);
    }
}

// A block of NWV waves owns 16 G output columns; wave w takes the 32-value
// K steps w, w + NWV, ...  In a step, lane (kq = l / 16, r16 = l % 16) loads
// values 8 kq .. 8 kq + 7 of weight row n0 + 16 g + r16 and of activation
// row r16: both operands put the same k in the same slot.
template <int G, int U, int NWV>
__global__ __launch_bounds__(NWV * 64) void bf16_skinny_kernel(const uint16_t* __restrict__ w,
                                                               const uint16_t* __restrict__ x,
                                                               void* __restrict__ out, int out_bf16, int M, int64_t N,
                                                               int64_t K, float alpha, Epilogue epi) {
  static_assert(NWV >= 4, "the final sum uses four waves");
  __shared__ v4f red[NWV][G][kWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const int64_t n0 = int64_t(blockIdx.x) * 16 * G;

  const uint16_t* wrow[G];
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

  const int64_t nsteps = (K + 31) / 32;
  for (int64_t s0 = wid; s0 < nsteps; s0 += int64_t(NWV) * U) {
    u32x4 wv[U][G];
    u32x4 xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kb = (s0 + int64_t(u) * NWV) * 32 + kq * 8;
      const bool ok = kb < K;  // K % 8 == 0: a chunk is wholly inside or outside
#pragma unroll
      for (int g = 0; g < G; ++g) wv[u][g] = ok ? ld16_stream(wrow[g] + kb) : u32x4{0u, 0u, 0u, 0u};
      xv[u] = ok && xrow_ok ? ld16(xrow + kb) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const v8bf a = __builtin_bit_cast(v8bf, xv[u]);
#pragma unroll
      for (int g = 0; g < G; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, wv[u][g]), acc[g], 0, 0, 0);
    }
  }

#pragma unroll
  for (int g = 0; g < G; ++g) red[wid][g][lane] = acc[g];
  __syncthreads();

  // Thread (wid, lane) of the first four waves finishes accumulator element
  // v = wid of every lane: D[i][j] with i = m = 4 (lane / 16) + wid and
  // j = column n0 + 16 g + lane % 16.
  if (wid >= 4) return;
  const int m = 4 * (lane >> 4) + wid;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NWV; ++q) s += red[q][g][lane][wid];
    const int64_t n = n0 + 16 * g + r16;
    if (m < M && n < N) store_epi(out, m, n, N, s, alpha, out_bf16, epi);
  }
}

template <int M, int ROWS>
hipError_t launch_gemv_rows(bool wide, const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t N,
                            int64_t K, float alpha, const Epilogue& epi, hipStream_t s) {
  constexpr int kThreads = 256;
  constexpr int kRowsPerBlock = ROWS * (kThreads / kWave);
  const int64_t blocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  if (!wide)
    return launch(bf16_gemv_any_kernel<M, ROWS>, dim3(blocks), dim3(kThreads), 0, s, w, x, out, out_bf16, N, K,
                  alpha, epi);
  // Rows of 512 or more chunks keep four chunks per lane in flight at M = 1.
  const int64_t per_lane = ((K >> 3) + kWave - 1) / kWave;
  if (M > 1 || per_lane <= 2)
    return launch(bf16_gemv_wide_kernel<M, ROWS, 2>, dim3(blocks), dim3(kThreads), 0, s, w, x, out, out_bf16, N, K,
                  alpha, epi);
  return launch(bf16_gemv_wide_kernel<M, ROWS, 4>, dim3(blocks), dim3(kThreads), 0, s, w, x, out, out_bf16, N, K,
                alpha, epi);
}

template <int M>
hipError_t launch_gemv_m(bool wide, const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t N,
                         int64_t K, float alpha, int num_cus, const Epilogue& epi, hipStream_t s) {
  if (N >= int64_t(num_cus) * 16) return launch_gemv_rows<M, 2>(wide, w, x, out, out_bf16, N, K, alpha, epi, s);
  return launch_gemv_rows<M, 1>(wide, w, x, out, out_bf16, N, K, alpha, epi, s);
}

template <int G, int U, int NWV>
hipError_t launch_skinny(const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                         int64_t K, float alpha, const Epilogue& epi, hipStream_t s) {
  const int64_t blocks = (N + 16 * G - 1) / (16 * G);
  return launch(bf16_skinny_kernel<G, U, NWV>, dim3(blocks), dim3(NWV * kWave), 0, s, w, x, out, out_bf16, int(M),
                N, K, alpha, epi);
}

}  // namespace

bool bf16_wide(const void* w, const void* x, int64_t K) {
  return K % 8 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
}

hipError_t launch_bf16_gemv(const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                            int64_t K, float alpha, int num_cus, hipStream_t s, const Epilogue& epi) {
  const bool wide = bf16_wide(w, x, K);
  switch (M) {
    case 1: return launch_gemv_m<1>(wide, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 2: return launch_gemv_m<2>(wide, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 3: return launch_gemv_m<3>(wide, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 4: return launch_gemv_m<4>(wide, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bf16_skinny(const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                              int64_t K, float alpha, int num_cus, hipStream_t s, const Epilogue& epi) {
  if (M < 1 || M > 16 || !bf16_wide(w, x, K)) return hipErrorInvalidValue;
  // The FP8 skinny kernel's choice: four 16-column groups per block from
  // 8192 output features, else one group with more K steps in flight.
  (void)num_cus;
  if (N >= 8192) return launch_skinny<4, 2, 16>(w, x, out, out_bf16, M, N, K, alpha, epi, s);
  return launch_skinny<1, 4, 16>(w, x, out, out_bf16, M, N, K, alpha, epi, s);
}

}  // namespace qlinear
