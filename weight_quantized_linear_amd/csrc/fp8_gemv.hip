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

// The 16 bytes at offset s (0 .. 15) of the 32-byte window lo:hi, as four
// dwords (s is uniform over the wave, so the dword select is a scalar branch;
// v_alignbyte takes the byte shift within a dword).
__device__ __forceinline__ u32x4 window16(const u32x4& lo, const u32x4& hi, int s) {
  uint32_t d0, d1, d2, d3, d4;
  switch (s >> 2) {
    case 0: d0 = lo.x; d1 = lo.y; d2 = lo.z; d3 = lo.w; d4 = hi.x; break;
    case 1: d0 = lo.y; d1 = lo.z; d2 = lo.w; d3 = hi.x; d4 = hi.y; break;
    case 2: d0 = lo.z; d1 = lo.w; d2 = hi.x; d3 = hi.y; d4 = hi.z; break;
    default: d0 = lo.w; d1 = hi.x; d2 = hi.y; d3 = hi.z; d4 = hi.w; break;
  }
  const uint32_t b = uint32_t(s & 3);
  return u32x4{__builtin_amdgcn_alignbyte(d1, d0, b), __builtin_amdgcn_alignbyte(d2, d1, b),
               __builtin_amdgcn_alignbyte(d3, d2, b), __builtin_amdgcn_alignbyte(d4, d3, b)};
}

// Bytes 0 .. keep-1 of a dword (keep clamped to 0 .. 4).
__device__ __forceinline__ uint32_t keep_bytes(uint32_t v, int keep) {
  return keep >= 4 ? v : keep <= 0 ? 0u : v & ((1u << (8 * keep)) - 1u);
}

// Any K and any weight alignment, activation rows 16-byte aligned: rows of
// K bytes start at arbitrary byte offsets (K = 2050, or a weight view), so
// lane `l` still owns the 16 values k = 16c .. 16c + 15 of each row (c = l,
// l + 64, ...) and reads them with 16-byte loads: the aligned block at or
// below the first byte, plus the next block when the row's start offset is
// not zero, shifted into place by window16.  Every load lies in an aligned
// block that holds a byte of the row (never past the weight's last 16-byte
// block).  In the row's last chunk the weight bytes and activation values
// past K are zeroed before use: a byte of the next row could decode to NaN,
// and 0 x NaN would poison the sum.
template <int M, int ROWS, int U>
__global__ __launch_bounds__(256) void fp8_gemv_shift_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, void* __restrict__ out,
    int out_bf16, int64_t N, int64_t K, float alpha, Epilogue epi) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t row0 = wave * ROWS;
  if (row0 >= N) return;  // uniform per wave

  const int64_t nk = (K + 15) >> 4;
  const uint8_t* base[ROWS];  // aligned block at or below the row's first byte
  int sh[ROWS];               // row start - base, 0 .. 15 (uniform)
  int64_t last[ROWS];         // offset from base of the last aligned block holding a byte of the row
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int64_t row = row0 + r < N ? row0 + r : N - 1;  // tail rows re-read the last row, never stored
    const uintptr_t b = reinterpret_cast<uintptr_t>(w) + uintptr_t(row * K);
    base[r] = reinterpret_cast<const uint8_t*>(b & ~uintptr_t(15));
    sh[r] = int(b & 15);
    last[r] = int64_t(((b + uintptr_t(K) - 1) & ~uintptr_t(15)) - (b & ~uintptr_t(15)));
  }

  float acc[M][ROWS];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[m][r] = 0.f;

  const u32x4 zero{0u, 0u, 0u, 0u};
  for (int64_t c0 = 0; c0 < nk; c0 += int64_t(kWave) * U) {
    u32x4 lo[U][ROWS], hi[U][ROWS];
    u32x4 xv[U][M][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + int64_t(u) * kWave + lane;
      const bool ok = c < nk;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        lo[u][r] = ok ? ld16_stream(base[r] + c * 16) : zero;
        hi[u][r] = ok && sh[r] != 0 && c * 16 + 16 <= last[r] ? ld16_stream(base[r] + c * 16 + 16) : zero;
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint16_t* xp = x + m * K + c * 16;
        xv[u][m][0] = ok ? ld16(xp) : zero;
        xv[u][m][1] = ok && c * 16 + 8 < K ? ld16(xp + 8) : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + int64_t(u) * kWave + lane;
      const int rem = int(K - c * 16 < 16 ? K - c * 16 : 16);  // values of this chunk inside the row
      u32x4 wv[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) wv[r] = window16(lo[u][r], hi[u][r], sh[r]);
      if (rem < 16) {  // the row's last chunk (or a chunk past it: rem <= 0 clears it all)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          wv[r].x = keep_bytes(wv[r].x, rem);
          wv[r].y = keep_bytes(wv[r].y, rem - 4);
          wv[r].z = keep_bytes(wv[r].z, rem - 8);
          wv[r].w = keep_bytes(wv[r].w, rem - 12);
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int h = 0; h < 2; ++h) {  // two bfloat16 values per dword
            xv[u][m][h].x = keep_bytes(xv[u][m][h].x, 2 * (rem - 8 * h));
            xv[u][m][h].y = keep_bytes(xv[u][m][h].y, 2 * (rem - 8 * h - 2));
            xv[u][m][h].z = keep_bytes(xv[u][m][h].z, 2 * (rem - 8 * h - 4));
            xv[u][m][h].w = keep_bytes(xv[u][m][h].w, 2 * (rem - 8 * h - 6));
          }
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {  // dword d of the chunk = values 4d .. 4d+3
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const v2bf w01 = __builtin_bit_cast(v2bf, e4m3x2_to_bf16x2<false>(wv[r][d]));
          const v2bf w23 = __builtin_bit_cast(v2bf, e4m3x2_to_bf16x2<true>(wv[r][d]));
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

// Weight loads: 0 = one byte per lane, 1 = 16-byte aligned rows, 2 = 16-byte
// loads shifted into place (rows at any byte offset).
enum { kBytes = 0, kWide = 1, kShift = 2 };

template <int M, int ROWS>
hipError_t launch_rows(int mode, const uint8_t* w, const uint16_t* x, void* out, int out_bf16,
                       int64_t N, int64_t K, float alpha, const Epilogue& epi, hipStream_t s) {
  constexpr int kThreads = 256;
  constexpr int kRowsPerBlock = ROWS * (kThreads / kWave);
  const int64_t blocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  if (mode == kShift) {
    // Up to two block loads per 16 values: U = 3 keeps about as many loads
    // in flight as the wide kernel's U = 4, and one pass covers rows of up to
    // 3072 values (K = 2050 included).
    if constexpr (M == 1) {
      if ((((K + 15) >> 4) + kWave - 1) / kWave > 2)
        return launch(fp8_gemv_shift_kernel<M, ROWS, 3>, dim3(blocks), dim3(kThreads), 0, s, w, x, out,
                      out_bf16, N, K, alpha, epi);
    }
    return launch(fp8_gemv_shift_kernel<M, ROWS, 2>, dim3(blocks), dim3(kThreads), 0, s, w, x, out,
                  out_bf16, N, K, alpha, epi);
  }
  if (mode == kWide) {
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
hipError_t launch_m(int mode, const uint8_t* w, const uint16_t* x, void* out, int out_bf16,
                    int64_t N, int64_t K, float alpha, int num_cus, const Epilogue& epi, hipStream_t s) {
  // Two rows per wave once that still gives every SIMD several waves.  (One
  // row per wave at N = 4096, or K split over four waves per row at N =
  // 4096, K = 14336, measured the same or slower: 4.9 vs 4.9 us, 15.9 vs
  // 12.5 us.)
  if (N >= int64_t(num_cus) * 16) return launch_rows<M, 2>(mode, w, x, out, out_bf16, N, K, alpha, epi, s);
  return launch_rows<M, 1>(mode, w, x, out, out_bf16, N, K, alpha, epi, s);
}

}  // namespace

hipError_t launch_fp8_gemv(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M,
                           int64_t N, int64_t K, float alpha, int num_cus, hipStream_t s, const Epilogue& epi) {
  // The shifted loads need every activation row 16-byte aligned.
  const bool x_rows = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (M == 1 || K % 8 == 0);
  const int mode = !x_rows ? kBytes
                   : (K % 16 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0) ? kWide
                                                                                : kShift;
  switch (M) {
    case 1: return launch_m<1>(mode, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 2: return launch_m<2>(mode, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 3: return launch_m<3>(mode, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    case 4: return launch_m<4>(mode, w, x, out, out_bf16, N, K, alpha, num_cus, epi, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlinear
