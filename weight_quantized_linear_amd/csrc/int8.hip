// W8A8 int8: the per-row activation quantiser and the int8 x int8 -> int32
// matrix-core GEMM with the dequantising epilogue.
//
// What is computed ("int8_matmul" page, "Quantization (W8A8)" and summary):
// both operands are symmetric absmax int8 with scale = absmax / 127, the
// activation per row (quantised online by a separate one-pass kernel), the
// weight per output channel (pre-quantised); raw products accumulate in
// int32; the epilogue multiplies each output by a_scale[row] * b_scale[col],
// adds the optional per-column bias after the dequantisation and casts to
// bfloat16.
//
// Quantiser (gfx950): one wave per row.  A row of up to 4096 values is read
// once into registers (16-byte loads, all issued at once); the absmax is a
// wave-wide max over the values' magnitude bits (so that a NaN or an
// infinity reaches it); the codes are q = round-half-even(x / scale),
// clamped to +-127, produced from the registers, with the quotient taken
// from a once-per-row reciprocal and two fma corrections, which gives the
// codes of the IEEE float32 division exactly (quantize_rcp; rows with a
// subnormal scale divide).  An all-zero row gives scale 0 and zero codes; a
// row with a NaN or an infinity gives scale NaN or +inf and zero codes.
// Longer rows are read a second time for the quantisation pass.
//
// GEMM: K % 64 == 0 with aligned operands runs the pipelined direct-to-LDS
// kernel of gemm_lds.hip.  This file's kernel serves every other shape: a
// 256-thread block computes a 128 x 128 int32 tile in 128-byte K strips
// staged in LDS through registers (zero-filled past K); four waves (2 x 2,
// 64 x 64) each run 4 x 4 v_mfma_i32_16x16x64_i8 per 64-byte K step.
#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

namespace {

// ---------------------------------------------------------------- quantiser

// |x| of a bfloat16 as its magnitude bits: for non-negative values the bit
// patterns order like the values, with +inf above every finite value and
// NaN above +inf, so an integer max over them is an absmax that a NaN or an
// infinity reaches (fmaxf would drop a NaN).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, uint32_t(__shfl_xor(int(v), off, kWave)));
  return v;
}

// Max of the magnitude bits of the two bfloat16 values in each dword.
__device__ __forceinline__ uint32_t abs_bits_max(uint32_t m, uint32_t v) {
  return max(max(m, v & 0x7FFFu), (v >> 16) & 0x7FFFu);
}

// Quantise with this row's scale when it is usable: a finite, positive
// absmax.  A zero row, or one holding a NaN (absmax NaN) or an infinity
// (absmax +inf: every quotient 0 or NaN), gets zero codes.
__device__ __forceinline__ bool amax_usable(uint32_t amax_bits) { return amax_bits - 1u < 0x7F80u - 1u; }

__device__ __forceinline__ int8_t quantize_one(float x, float scale) {
  float q = rintf(x / scale);  // IEEE division, round half to even
  q = fminf(fmaxf(q, -127.f), 127.f);
  return int8_t(int(q));
}

// Fast path: K % 8 == 0, x 16-byte aligned, q 8-byte aligned.
template <int CHUNKS>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ x,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ a_scale, int64_t M,
                                                            int64_t K) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= M) return;
  const uint16_t* xr = x + row * K;
  int8_t* qr = q + row * K;
  const int64_t nchunks = K >> 3;  // 8 elements per 16-byte chunk
  const bool fits = nchunks <= int64_t(kWave) * CHUNKS;

  u32x4 v[CHUNKS];
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int64_t c = int64_t(i) * kWave + lane;
    v[i] = c < nchunks ? ld16(xr + c * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  for (int64_t c0 = 0; c0 < nchunks; c0 += int64_t(kWave) * CHUNKS) {
    if (c0 > 0) {
#pragma unroll
      for (int i = 0; i < CHUNKS; ++i) {
        const int64_t c = c0 + int64_t(i) * kWave + lane;
        v[i] = c < nchunks ? ld16(xr + c * 8) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) amax_bits = abs_bits_max(amax_bits, v[i][d]);
    if (fits) break;
  }
  amax_bits = wave_max_u32(amax_bits);
  const float scale = __uint_as_float(amax_bits << 16) / 127.f;
  const bool usable = amax_usable(amax_bits);
  if (lane == 0) a_scale[row] = scale;
  for (int64_t c0 = 0; c0 < nchunks; c0 += int64_t(kWave) * CHUNKS) {
    if (!fits) {
#pragma unroll
      for (int i = 0; i < CHUNKS; ++i) {
        const int64_t c = c0 + int64_t(i) * kWave + lane;
        v[i] = c < nchunks ? ld16(xr + c * 8) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int64_t c = c0 + int64_t(i) * kWave + lane;
      if (c >= nchunks) continue;
      uint32_t packed[2] = {0u, 0u};
      if (usable) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t lo = uint8_t(quantize_one(bf16lo(v[i][d]), scale));
          const uint32_t hi = uint8_t(quantize_one(bf16hi(v[i][d]), scale));
          packed[d >> 1] |= (lo | (hi << 8)) << (16 * (d & 1));
        }
      }
      *reinterpret_cast<u32x2*>(qr + c * 8) = u32x2{packed[0], packed[1]};
    }
    if (fits) break;
  }
}

// q = clamp(rint(x / s), +-127) from r = 1/s (correctly rounded, once per
// row): q0 = x r, e = x - q0 s (exact, one fma), q1 = q0 + e r (one fma) is
// the correctly rounded quotient x / s wherever that quotient is a normal
// float32 (Markstein's correction step), and tiny quotients round to code 0
// either way, so the codes equal those of the IEEE division.  Checked on the
// CPU over every finite bfloat16 x for 3000 random and edge-case normal
// scales (exact rational arithmetic where float64 emulation could double
// round); rows with a subnormal scale keep the division.
__device__ __forceinline__ int8_t quantize_rcp(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  const float q1 = __builtin_fmaf(e, r, q0);
  const float q = fminf(fmaxf(rintf(q1), -127.f), 127.f);
  return int8_t(int(q));
}

// Rows of up to 512 CH values (K % 8 == 0, x 16-byte and q 8-byte
// aligned): a wave owns R consecutive rows and issues all R x CH 16-byte
// loads of them before it reduces or quantises any, so that the second
// row's data streams in while the first is quantised and stored.
template <int CH, int R>
__global__ __launch_bounds__(256) void quantize_rows_pipe_kernel(const uint16_t* __restrict__ x,
                                                                 int8_t* __restrict__ q,
                                                                 float* __restrict__ a_scale, int64_t M,
                                                                 int64_t K) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row0 = (int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave)) * R;
  if (row0 >= M) return;
  const int64_t nchunks = K >> 3;  // 8 elements per 16-byte chunk, at most 64 CH
  u32x4 v[R][CH];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t c = int64_t(i) * kWave + lane;
      v[r][i] = row0 + r < M && c < nchunks ? ld16(x + (row0 + r) * K + c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r;
    if (row >= M) break;  // uniform
    uint32_t amax_bits = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) amax_bits = abs_bits_max(amax_bits, v[r][i][d]);
    amax_bits = wave_max_u32(amax_bits);
    const float scale = __uint_as_float(amax_bits << 16) / 127.f;
    if (lane == 0) a_scale[row] = scale;
    const bool usable = amax_usable(amax_bits);
    const bool normal = scale >= 0x1p-126f;  // 1 / scale finite, quotients in the normal range
    const float rcp = 1.f / scale;
    int8_t* qr = q + row * K;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t c = int64_t(i) * kWave + lane;
      if (c >= nchunks) continue;
      uint32_t packed[2] = {0u, 0u};
      if (usable) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float lo = bf16lo(v[r][i][d]), hi = bf16hi(v[r][i][d]);
          const uint32_t ql = uint8_t(normal ? quantize_rcp(lo, scale, rcp) : quantize_one(lo, scale));
          const uint32_t qh = uint8_t(normal ? quantize_rcp(hi, scale, rcp) : quantize_one(hi, scale));
          packed[d >> 1] |= (ql | (qh << 8)) << (16 * (d & 1));
        }
      }
      *reinterpret_cast<u32x2*>(qr + c * 8) = u32x2{packed[0], packed[1]};
    }
  }
}

// Any K, any alignment: element-wise, two passes over the row.
__global__ __launch_bounds__(256) void quantize_rows_any_kernel(const uint16_t* __restrict__ x,
                                                                int8_t* __restrict__ q,
                                                                float* __restrict__ a_scale, int64_t M,
                                                                int64_t K) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= M) return;
  const uint16_t* xr = x + row * K;
  uint32_t amax_bits = 0;
  for (int64_t k = lane; k < K; k += kWave) amax_bits = max(amax_bits, uint32_t(xr[k] & 0x7FFFu));
  amax_bits = wave_max_u32(amax_bits);
  const float scale = __uint_as_float(amax_bits << 16) / 127.f;
  const bool usable = amax_usable(amax_bits);
  if (lane == 0) a_scale[row] = scale;
  for (int64_t k = lane; k < K; k += kWave)
    q[row * K + k] = usable ? quantize_one(bf16_to_f32(xr[k]), scale) : int8_t(0);
}

// ---------------------------------------------------------------- GEMM

constexpr int BM = 128, BN = 128, BK = 128;  // BK in bytes = int8 elements
constexpr int kThreads = 256;
constexpr int kLdsRow = BK + 16;
constexpr int kLdsTile = 128 * kLdsRow;

struct I8Operand {
  const int8_t* p;  // [rows, K]
  int64_t rows, K;
  bool vec;         // K % 16 == 0 and 16-byte aligned base
};

struct I8Stage { u32x4 v[4]; };

// Thread t loads chunks id = t + 256 i (i < 4): row id / 8, bytes 16 (id % 8) .. +15.
__device__ __forceinline__ void i8_load(const I8Operand& A, int64_t r0, int64_t k0, I8Stage& st, bool stream) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = threadIdx.x + kThreads * i;
    const int64_t r = r0 + (id >> 3);
    const int64_t k = k0 + 16 * (id & 7);
    if (r < A.rows && A.vec && k + 16 <= A.K) {
      st.v[i] = stream ? ld16_stream(A.p + r * A.K + k) : ld16(A.p + r * A.K + k);
    } else {
      uint32_t e[4] = {0u, 0u, 0u, 0u};
      if (r < A.rows) {
        for (int j = 0; j < 16; ++j)
          if (k + j < A.K) e[j >> 2] |= uint32_t(uint8_t(A.p[r * A.K + k + j])) << (8 * (j & 3));
      }
      st.v[i] = u32x4{e[0], e[1], e[2], e[3]};
    }
  }
}

__device__ __forceinline__ void i8_store(char* lds, const I8Stage& st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = threadIdx.x + kThreads * i;
    *reinterpret_cast<u32x4*>(lds + (id >> 3) * kLdsRow + 16 * (id & 7)) = st.v[i];
  }
}

__device__ __forceinline__ void i8_tile_of_block(int64_t b, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                                 int64_t& tn) {
  constexpr int kXcd = 8, kGroupM = 8;
  const int64_t total = tiles_m * tiles_n;
  const int64_t q = total / kXcd, r = total % kXcd;
  const int64_t xcd = b % kXcd, local = b / kXcd;
  const int64_t t = xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  const int64_t group = kGroupM * tiles_n;
  const int64_t g = t / group;
  const int64_t first_m = g * kGroupM;
  const int64_t gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int64_t in_group = t % group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// The 128 x 128 tile at (m0, n0) of out[M, N] (M = A.rows, N = B.rows).
// out_mode: 0 = float32, 1 = bfloat16 (both dequantised), 2 = raw int32
// accumulators.  Every thread of the block calls it.
__device__ void int8_dense_tile(char* lds, const I8Operand& A, const I8Operand& B, const float* __restrict__ a_scale,
                                const float* __restrict__ b_scale, const uint16_t* __restrict__ bias,
                                void* __restrict__ out, int out_mode, int64_t m0, int64_t n0) {
  char* lds_a = lds;
  char* lds_b = lds + kLdsTile;
  const int64_t M = A.rows, N = B.rows;

  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int wy = wid >> 1, wx = wid & 1;
  const int r16 = lane & 15, kq = lane >> 4;

  v4i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  I8Stage sa, sb;
  const int64_t nk = (A.K + BK - 1) / BK;
  i8_load(A, m0, 0, sa, false);
  i8_load(B, n0, 0, sb, true);
  for (int64_t kt = 0; kt < nk; ++kt) {
    __syncthreads();
    i8_store(lds_a, sa);
    i8_store(lds_b, sb);
    __syncthreads();
    if (kt + 1 < nk) {
      i8_load(A, m0, (kt + 1) * BK, sa, false);
      i8_load(B, n0, (kt + 1) * BK, sb, true);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i a[4], b[4];
      const int koff = ks * 64 + kq * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const v4i*>(lds_a + (wy * 64 + 16 * i + r16) * kLdsRow + koff);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const v4i*>(lds_b + (wx * 64 + 16 * j + r16) * kLdsRow + koff);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // acc[i][j][v] = C[m0 + 64 wy + 16 i + 4 kq + v][n0 + 64 wx + 16 j + r16]
  float bs[4], bb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wx * 64 + 16 * j + r16;
    bs[j] = (out_mode != 2 && n < N) ? b_scale[n] : 0.f;
    bb[j] = (out_mode != 2 && bias && n < N) ? bf16_to_f32(bias[n]) : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + wy * 64 + 16 * i + 4 * kq + v;
      if (m >= M) continue;
      const float as = out_mode != 2 ? a_scale[m] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wx * 64 + 16 * j + r16;
        if (n >= N) continue;
        const int32_t a32 = acc[i][j][v];
        if (out_mode == 2) {
          reinterpret_cast<int32_t*>(out)[m * N + n] = a32;
        } else {
          const float val = float(a32) * as * bs[j] + bb[j];
          if (out_mode == 1) reinterpret_cast<uint16_t*>(out)[m * N + n] = f32_to_bf16(val);
          else reinterpret_cast<float*>(out)[m * N + n] = val;
        }
      }
    }
}

__global__ __launch_bounds__(kThreads) void int8_gemm_kernel(I8Operand A, I8Operand B,
                                                             const float* __restrict__ a_scale,
                                                             const float* __restrict__ b_scale,
                                                             const uint16_t* __restrict__ bias,
                                                             void* __restrict__ out, int out_mode) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kLdsTile];
  int64_t tm, tn;
  i8_tile_of_block(blockIdx.x, (A.rows + BM - 1) / BM, (B.rows + BN - 1) / BN, tm, tn);
  int8_dense_tile(lds, A, B, a_scale, b_scale, bias, out, out_mode, tm * BM, tn * BN);
}

// Grouped W8A8 for any K and alignment: group z = blockIdx.z covers rows
// a_offsets[z] .. a_offsets[z+1]-1 (clipped to T) with expert expert_ids[z];
// blockIdx.x is the column tile and the group's row tiles are taken
// blockIdx.y, + gridDim.y, ...  An id outside 0 .. E-1 writes zeros.
__global__ __launch_bounds__(kThreads) void int8_grouped_any_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, const float* __restrict__ a_scale,
    const float* __restrict__ b_scale, const uint16_t* __restrict__ bias, const uint32_t* __restrict__ a_offsets,
    const int32_t* __restrict__ expert_ids, void* __restrict__ out, int out_mode, int64_t T, int64_t N, int64_t K,
    int64_t E, bool vec) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kLdsTile];
  const int64_t z = blockIdx.z;
  int64_t start = a_offsets[z], end = a_offsets[z + 1];
  start = start < T ? start : T;
  end = end < T ? end : T;
  if (end <= start) return;
  const int64_t rows = end - start;
  const int64_t e = expert_ids[z];
  const int64_t n0 = int64_t(blockIdx.x) * BN;
  const int es = out_mode == 1 ? 2 : 4;
  char* gout = static_cast<char*>(out) + start * N * es;
  for (int64_t mt = blockIdx.y; mt * BM < rows; mt += gridDim.y) {
    const int64_t m0 = mt * BM;
    if (e < 0 || e >= E) {
      for (int idx = threadIdx.x; idx < BM * BN; idx += kThreads) {
        const int64_t m = m0 + idx / BN, n = n0 + idx % BN;
        if (m >= rows || n >= N) continue;
        if (out_mode == 2) reinterpret_cast<int32_t*>(gout)[m * N + n] = 0;
        else if (out_mode == 1) reinterpret_cast<uint16_t*>(gout)[m * N + n] = 0;
        else reinterpret_cast<float*>(gout)[m * N + n] = 0.f;
      }
      continue;
    }
    const I8Operand A{a + start * K, rows, K, vec}, B{b + e * N * K, N, K, vec};
    int8_dense_tile(lds, A, B, a_scale ? a_scale + start : nullptr, b_scale ? b_scale + e * N : nullptr, bias ? bias + e * N : nullptr,
                    gout, out_mode, m0, n0);
  }
}

}  // namespace

hipError_t launch_int8_quantize(const uint16_t* x, int8_t* q, float* a_scale, int64_t M, int64_t K,
                                hipStream_t s) {
  const bool vec = (K % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(q) % 8 == 0);
  const int64_t blocks = (M + 3) / 4;
  if (!vec) return launch(quantize_rows_any_kernel, dim3(blocks), dim3(256), 0, s, x, q, a_scale, M, K);
  // One row per wave: with two or four rows a wave the launch has fewer
  // waves to cover the load latency (4096 x 3072: 8.7 us at one row, 10.4
  // at two, 14.2 at four).
  constexpr int R = 1;
  const int64_t pblocks = (M + 4 * R - 1) / (4 * R);
  const int64_t ch = ((K >> 3) + kWave - 1) / kWave;  // 16-byte chunks per lane
  if (ch <= 2) return launch(quantize_rows_pipe_kernel<2, R>, dim3(pblocks), dim3(256), 0, s, x, q, a_scale, M, K);
  if (ch <= 4) return launch(quantize_rows_pipe_kernel<4, R>, dim3(pblocks), dim3(256), 0, s, x, q, a_scale, M, K);
  if (ch <= 6) return launch(quantize_rows_pipe_kernel<6, R>, dim3(pblocks), dim3(256), 0, s, x, q, a_scale, M, K);
  if (ch <= 8) return launch(quantize_rows_pipe_kernel<8, R>, dim3(pblocks), dim3(256), 0, s, x, q, a_scale, M, K);
  return launch(quantize_rows_kernel<8>, dim3(blocks), dim3(256), 0, s, x, q, a_scale, M, K);
}

hipError_t launch_int8_gemm(const int8_t* a, const int8_t* b, const float* a_scale, const float* b_scale,
                            const uint16_t* bias, void* out, int out_mode, int64_t M, int64_t N, int64_t K,
                            int num_cus, hipStream_t s) {
  if (int8_lds_supported(a, b, M, N, K))
    return launch_int8_gemm_lds(a, b, a_scale, b_scale, bias, out, out_mode, M, N, K, num_cus, s);
  const bool vec = (K % 16 == 0) && (reinterpret_cast<uintptr_t>(a) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(b) % 16 == 0);
  const I8Operand A{a, M, K, vec}, B{b, N, K, vec};
  const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return launch(int8_gemm_kernel, dim3(blocks), dim3(kThreads), 0, s, A, B, a_scale, b_scale, bias, out,
                out_mode);
}

hipError_t launch_int8_grouped(const int8_t* a, const int8_t* b, const float* a_scale, const float* b_scale,
                               const uint16_t* bias, const uint32_t* a_offsets, const int32_t* expert_ids, void* out,
                               int out_mode, int64_t G, int64_t max_tokens, int64_t E, int64_t T, int64_t N, int64_t K,
                               int num_cus, hipStream_t s) {
  if (int8_grouped_lds_supported(a, b, G, T, N, K))
    return launch_int8_grouped_lds(a, b, a_scale, b_scale, bias, a_offsets, expert_ids, out, out_mode, G, E, T, N, K,
                                   num_cus, s);
  // vec needs every expert's rows 16-byte aligned: K % 16 == 0 and aligned bases.
  const bool vec = (K % 16 == 0) && (reinterpret_cast<uintptr_t>(a) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(b) % 16 == 0);
  int64_t tiles_m = (max_tokens + BM - 1) / BM;
  if (tiles_m < 1) tiles_m = 1;
  if (tiles_m > 65535) tiles_m = 65535;
  return launch(int8_grouped_any_kernel, dim3((N + BN - 1) / BN, tiles_m, G), dim3(kThreads), 0, s, a, b, a_scale,
                b_scale, bias, a_offsets, expert_ids, out, out_mode, T, N, K, E, vec);
}

}  // namespace qlinear
