// W8A16 skinny GEMM on the matrix cores, 1 <= M <= 16:
//     out[m, n] = alpha * sum_k x[m, k] * dec(W[n, k])
//
// What is computed is the "Matmul2dFp8" page's W8A16 GEMM (bf16 activation,
// float8_e4m3fn weight, float32 accumulation).  At M <= 16 the product is
// still bound by the weight read, but M multiply-adds per weight byte exceed
// what the vector ALU can sustain at full HBM bandwidth, so the products run
// on the matrix cores.  The E4M3 -> bf16 widening is exact, so the matrix
// cores see exactly the decoded weight; accumulation is float32.
//
// Six kernels, chosen by shape (all measured on the decode shapes):
//
// * fp8_skinny_kernel (v_mfma_f32_16x16x32_bf16): a block of NWV waves owns
//   16*G output columns; its waves take interleaved 64-byte K steps, each
//   lane loading one 16-byte chunk per 16-row group per step (row l % 16,
//   bytes 16*(l/16) .. +15 of the step); the M activation rows (zero-padded
//   to 16) are the other operand and the NWV partial accumulators are summed
//   through LDS at the end.
// * fp8_skinny_lds_kernel: the same matrix-core work, but the block first
//   reads a 64-row x 512-byte weight tile with fully contiguous 16-byte loads
//   (64 lanes over 1 KiB of two rows) into LDS and the waves take their
//   operands from there; on the 128256-row weight this beats reading the
//   operand layout straight from HBM (106 vs 120 us at M = 16).
// * fp8_skinny4_kernel (v_mfma_f32_4x4x4bf16_1k, M <= 4): the instruction is
//   16 independent 4x4x4 products, one per group of four lanes, so lane
//   4b + j can read 16 contiguous bytes of weight row j at offset 16b: one
//   load instruction covers four rows x 256 contiguous bytes.  Block b of the
//   instruction accumulates the k-range 16b .. of every step, and the 16
//   block partials are summed across lanes at the end.
// * fp8_skinny_xlds_kernel (the same instruction, M <= 8, K % 256 == 0): the
//   activation is copied to LDS once per block and every wave streams whole
//   4 KiB weight row segments; described at the kernel.
// * fp8_skinny_stream_kernel (16x16x32, K up to 4096, N >= 8192 for
//   5 <= M <= 16 and 8192 <= N < 65536 for 3 <= M <= 4): whole weight rows
//   DMA'd into an LDS ring, the activation held in registers; described at
//   the kernel.
// * fp8_skinny_splitk_kernel (16x16x32, long K): K slices over blocks into
//   float32 partial planes of the caller's workspace.
//
// In every kernel the same k-slot assignment is used for both operands, so
// the pairing of activation and weight elements does not depend on how the
// matrix core orders k-slots internally.
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

namespace {

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

template <int G, int U, int NWV, bool FUSED>
__global__ __launch_bounds__(NWV * 64) void fp8_skinny_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, void* __restrict__ out,
    int out_bf16, int M, int64_t N, int64_t K, float alpha, Epilogue epi) {
  constexpr int kWaves = NWV;
  static_assert(NWV >= 4, "the final sum uses four waves");
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
      for (int g = 0; g < G; ++g) wv[u][g] = ok ? ld16(wrow[g] + kb) : u32x4{0u, 0u, 0u, 0u};
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

  // Thread (wid, lane) of the first four waves finishes accumulator element
  // v = wid of every lane: D[i][j] with i = m = 4*(lane/16) + wid and
  // j = column n0 + 16g + lane%16.
  if (wid >= 4) return;
  const int m = 4 * (lane >> 4) + wid;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) s += red[q][g][lane][wid];
    const int64_t n = n0 + 16 * g + r16;
    if (m < M && n < N) store_maybe_epi<FUSED>(out, m, n, N, s, alpha, out_bf16, epi);
  }
}

// LDS-staged variant: block = 16*G rows x all of K in tiles of KT bytes per
// row.  Thread t loads chunk id = t + 256 i of the tile: row id / (KT/16),
// bytes 16 (id % (KT/16)), so one load instruction covers 1 KiB of
// contiguous weight.  Wave w then takes bytes [w KT/4, (w+1) KT/4) of every
// row of the tile in 64-byte matrix-core steps.  The next tile's loads are
// issued before the current tile's matrix-core work.
template <int G, int KT, bool FUSED>
__global__ __launch_bounds__(256) void fp8_skinny_lds_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, void* __restrict__ out,
    int out_bf16, int M, int64_t N, int64_t K, float alpha, Epilogue epi) {
  constexpr int kRow = KT + 16;                        // padded LDS row (bytes)
  constexpr int kChunksPerRow = KT / 16;
  constexpr int kLoads = 16 * G * kChunksPerRow / 256;  // 16-byte loads per thread per tile
  static_assert(kLoads * 256 == 16 * G * kChunksPerRow, "tile must split evenly over the block");
  __shared__ __attribute__((aligned(16))) char tile[16 * G * kRow];
  __shared__ v4f red[4][G][kWave];

  const int t = threadIdx.x, lane = t & (kWave - 1), wid = t / kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const int64_t n0 = int64_t(blockIdx.x) * 16 * G;
  const bool xrow_ok = r16 < M;
  const uint16_t* xrow = x + int64_t(xrow_ok ? r16 : 0) * K;

  v4f acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};

  u32x4 pre[kLoads];
  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int id = t + 256 * i;
      int64_t n = n0 + id / kChunksPerRow;
      if (n >= N) n = N - 1;
      const int64_t k = k0 + 16 * (id % kChunksPerRow);
      pre[i] = k < K ? ld16(w + n * K + k) : u32x4{0u, 0u, 0u, 0u};
    }
  };

  const int64_t ntiles = (K + KT - 1) / KT;
  load_tile(0);
  for (int64_t tt = 0; tt < ntiles; ++tt) {
    __syncthreads();  // previous tile's LDS reads are done
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int id = t + 256 * i;
      *reinterpret_cast<u32x4*>(tile + (id / kChunksPerRow) * kRow + 16 * (id % kChunksPerRow)) = pre[i];
    }
    __syncthreads();
    if (tt + 1 < ntiles) load_tile((tt + 1) * KT);
    constexpr int kSteps = KT / 4 / 64;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int kl = wid * (KT / 4) + 64 * s + 16 * kq;
      const int64_t kg = tt * KT + kl;
      const bool ok = kg < K && xrow_ok;
      const v8bf a0 = __builtin_bit_cast(v8bf, ok ? ld16(xrow + kg) : u32x4{0u, 0u, 0u, 0u});
      const v8bf a1 = __builtin_bit_cast(v8bf, ok ? ld16(xrow + kg + 8) : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const u32x4 wv = *reinterpret_cast<const u32x4*>(tile + (16 * g + r16) * kRow + kl);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, e4m3x8_to_bf16x8(wv.x, wv.y), acc[g], 0, 0, 0);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, e4m3x8_to_bf16x8(wv.z, wv.w), acc[g], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int g = 0; g < G; ++g) red[wid][g][lane] = acc[g];
  __syncthreads();
  const int m = 4 * (lane >> 4) + wid;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) s += red[q][g][lane][wid];
    const int64_t n = n0 + 16 * g + r16;
    if (m < M && n < N) store_maybe_epi<FUSED>(out, m, n, N, s, alpha, out_bf16, epi);
  }
}

// 4x4x4 variant for M <= 4: each wave owns 4*G rows and all of K; lane
// l = 4b + j loads weight row n0 + 4g + j and activation row j at byte/element
// offset 256 s + 16 b of every 256-wide K step s.
template <int G, int U, bool FUSED>
__global__ __launch_bounds__(256) void fp8_skinny4_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, void* __restrict__ out,
    int out_bf16, int M, int64_t N, int64_t K, float alpha, Epilogue epi) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t n0 = wave * 4 * G;
  if (n0 >= N) return;  // uniform per wave; no block-level synchronisation below
  const int b = lane >> 2, j = lane & 3;

  const uint8_t* wrow[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    int64_t n = n0 + 4 * g + j;
    if (n >= N) n = N - 1;
    wrow[g] = w + n * K;
  }
  const bool xok = j < M;
  const uint16_t* xrow = x + int64_t(xok ? j : 0) * K;

  v4f acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t nsteps = (K + 255) / 256;
  for (int64_t s0 = 0; s0 < nsteps; s0 += U) {
    u32x4 wv[U][G];
    u32x4 xv[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kb = (s0 + u) * 256 + 16 * b;
      const bool ok = kb < K;
#pragma unroll
      for (int g = 0; g < G; ++g) wv[u][g] = ok ? ld16_stream(wrow[g] + kb) : u32x4{0u, 0u, 0u, 0u};
      xv[u][0] = ok && xok ? ld16(xrow + kb) : u32x4{0u, 0u, 0u, 0u};
      xv[u][1] = ok && xok ? ld16(xrow + kb + 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // k = 16 b + 4 q .. +3 of the step
        const u32x4& xa = xv[u][q >> 1];
        const u32x2 xp = (q & 1) ? u32x2{xa.z, xa.w} : u32x2{xa.x, xa.y};
        const v4bf ax = __builtin_bit_cast(v4bf, xp);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint32_t d = wv[u][g][q];
          const u32x2 wp{e4m3x2_to_bf16x2<false>(d), e4m3x2_to_bf16x2<true>(d)};
          acc[g] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ax, __builtin_bit_cast(v4bf, wp), acc[g], 0, 0, 0);
        }
      }
  }

  // acc[g][i] in lane 4b + j = partial out[i][n0 + 4g + j] over block b's
  // k-range; sum the 16 blocks (lanes j, j + 4, ..., j + 60).
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[g][i];
      v += __shfl_xor(v, 4, kWave);
      v += __shfl_xor(v, 8, kWave);
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      acc[g][i] = v;
    }
  if (lane < 4) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t n = n0 + 4 * g + j;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < M) store_maybe_epi<FUSED>(out, i, n, N, acc[g][i], alpha, out_bf16, epi);
    }
  }
}

// One reduce-scatter step over lane bit `mask`: the lower lane keeps the
// sums of v[0 .. H), the upper lane those of v[H .. 2H), both in v[0 .. H).
template <int H>
__device__ __forceinline__ void rs_halve(float* v, int lane, int mask) {
  const bool upper = (lane & mask) != 0;
#pragma unroll
  for (int e = 0; e < H; ++e) {
    const float send = upper ? v[e] : v[e + H];
    const float keep = upper ? v[e + H] : v[e];
    v[e] = keep + __shfl_xor(send, mask, kWave);
  }
}

// Activation-resident variant (K % 256 == 0, the padded activation fits in
// LDS): v_mfma_f32_4x4x4bf16_1k again, but
// * a wave owns 4 weight rows at a time and streams 4 KiB of each row per
//   stage (16 loads of 16 bytes per lane, all issued before any is used), so
//   every stage requests whole 4 KiB row segments at once, the access that
//   keeps HBM near its peak;
// * the activation rows (zero-padded to 4 * MG) are copied once per block
//   into LDS in the order the matrix cores take them, so that they are read
//   from HBM/L2 once per block instead of once per weight chunk; 16-byte unit
//   ((c * MG + p) * 2 + h) * 64 + 4 b + j holds x[4 p + j][256 c + 16 b + 8 h
//   .. + 8], which lane 4 b + j reads with one conflict-free ds_read_b128;
// * the 16 instruction blocks' partial sums (one per 16-byte k offset b) are
//   combined with a reduce-scatter across lanes: each exchange halves the
//   values a lane holds, so 4 MG values take 4 MG - 1 exchanges, after which
//   lane 4 b + j holds one finished output.
// With KS == 1 every wave walks 4-row groups on its own with a grid stride.
// With few rows (KS > 1) the K chunks of a group are split over KS waves of
// the block, whose partial outputs are added through LDS in a fixed order;
// the block then walks NWB / KS groups per round.
template <int MG, int NWB, int KS, bool FUSED>
__global__ __launch_bounds__(NWB * 64) void fp8_skinny_xlds_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, void* __restrict__ out,
    int out_bf16, int M, int N, int K, float alpha, Epilogue epi) {
  extern __shared__ __attribute__((aligned(16))) char xs[];
  constexpr int kU = 16;          // 16-byte loads per lane per stage (4 KiB per row)
  constexpr int kV = 4 * MG;      // accumulator values per lane
  constexpr int kChains = 4 / MG; // independent accumulators per m-group
  constexpr int kLogV = MG == 1 ? 2 : (MG == 2 ? 3 : 4);
  constexpr int kGpb = NWB / KS;  // groups a block runs at once
  static_assert(MG == 1 || MG == 2 || MG == 4, "m-groups");
  static_assert(NWB % KS == 0, "whole groups per block");

  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int b = lane >> 2, j = lane & 3;
  const int gi = wid / KS, ks = wid % KS;
  const int nch = K >> 8;            // 256-wide k chunks (K % 256 == 0)
  const int groups = (N + 3) >> 2;   // 4-row weight groups
  const int c_lo = ks * nch / KS, c_hi = (ks + 1) * nch / KS;  // this wave's chunks
  const int gstride = gridDim.x * kGpb;

  u32x4 wv[kU];
  auto load_stage = [&](int grp, int c0) {
    const int n = min(4 * grp + j, N - 1);  // rows past N re-read the last row; never stored
    const uint8_t* wr = w + int64_t(n) * K + 16 * b;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      wv[u] = c0 + u < c_hi ? ld16_stream(wr + int64_t(c0 + u) * 256) : u32x4{0u, 0u, 0u, 0u};
  };

  // Partial out[m][4 grp + j] over this wave's chunks, for the lane that
  // ends up holding it (m = b >> (4 - kLogV)); the first stage is loaded.
  auto run_group = [&](int grp) {
    v4f acc[MG][kChains];
#pragma unroll
    for (int p = 0; p < MG; ++p)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[p][c] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int c0 = c_lo; c0 < c_hi; c0 += kU) {
      if (c0 > c_lo) load_stage(grp, c0);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (c0 + u < c_hi) {
          const char* xp = xs + (int64_t(c0 + u) * MG * 2 * 64 + lane) * 16;
          u32x4 xa[MG], xb[MG];
#pragma unroll
          for (int p = 0; p < MG; ++p) {
            xa[p] = *reinterpret_cast<const u32x4*>(xp + p * 2048);
            xb[p] = *reinterpret_cast<const u32x4*>(xp + p * 2048 + 1024);
          }
          // Weight k-quad q is decoded once and used by every m-group;
          // consecutive instructions go to different accumulators.
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t d = wv[u][q];
            const u32x2 bp{e4m3x2_to_bf16x2<false>(d), e4m3x2_to_bf16x2<true>(d)};
#pragma unroll
            for (int p = 0; p < MG; ++p) {
              const u32x4& xh = q < 2 ? xa[p] : xb[p];
              const u32x2 ap = (q & 1) ? u32x2{xh.z, xh.w} : u32x2{xh.x, xh.y};
              acc[p][q % kChains] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
                  __builtin_bit_cast(v4bf, ap), __builtin_bit_cast(v4bf, bp), acc[p][q % kChains], 0, 0, 0);
            }
          }
        }
      }
    }

    // v[4 p + e] = partial out[4 p + e][4 grp + j] over this lane's k offsets.
    float v[kV];
#pragma unroll
    for (int p = 0; p < MG; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float t = 0.f;
#pragma unroll
        for (int c = 0; c < kChains; ++c) t += acc[p][c][e];
        v[4 * p + e] = t;
      }
    // Reduce-scatter over the 16 blocks (lane bits 2..5, high bit first).
    rs_halve<kV / 2>(v, lane, 32);
    rs_halve<kV / 4>(v, lane, 16);
    if constexpr (kV >= 8) rs_halve<kV / 8>(v, lane, 8);
    else v[0] += __shfl_xor(v[0], 8, kWave);
    if constexpr (kV >= 16) rs_halve<1>(v, lane, 4);
    else v[0] += __shfl_xor(v[0], 4, kWave);
    return v[0];
  };
  // Lane 4 b + j holds out[b >> (4 - log2 V)][4 grp + j]; every
  // 2^(4 - log2 V)-th b stores.
  auto store = [&](int grp, float val) {
    const int m = b >> (4 - kLogV);
    const int n = 4 * grp + j;
    if ((b & ((1 << (4 - kLogV)) - 1)) == 0 && m < M && n < N) store_maybe_epi<FUSED>(out, m, n, N, val, alpha, out_bf16, epi);
  };

  int g = blockIdx.x * kGpb + gi;
  if (g < groups) load_stage(g, c_lo);

  // Activation -> LDS in operand order; rows past M are zeros.
  {
    const int units = nch * MG * 128;
    constexpr int kT = NWB * kWave, kBatch = 4;
    for (int base = threadIdx.x; base < units; base += kT * kBatch) {
      u32x4 v[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int u = base + t * kT;
        const int I = u >> 6, l = u & 63;
        const int h = I & 1, p = (I >> 1) % MG, c = (I >> 1) / MG;
        const int m = 4 * p + (l & 3);
        v[t] = u < units && m < M ? ld16(x + int64_t(m) * K + 256 * c + 16 * (l >> 2) + 8 * h)
                                  : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int u = base + t * kT;
        if (u < units) *reinterpret_cast<u32x4*>(xs + 16 * u) = v[t];
      }
    }
  }
  __syncthreads();

  if constexpr (KS == 1) {
    for (; g < groups; g += gstride) {
      const float val = run_group(g);
      store(g, val);
      if (g + gstride < groups) load_stage(g + gstride, c_lo);
    }
  } else {
    // Partial sums of the KS waves of a group meet in red[wid][lane], after
    // the activation copy.  The round loop bound is uniform over the block.
    float* red = reinterpret_cast<float*>(xs + int64_t(nch) * MG * 2048);
    for (int g0 = blockIdx.x * kGpb; g0 < groups; g0 += gstride) {
      g = g0 + gi;
      const float val = g < groups ? run_group(g) : 0.f;
      red[wid * kWave + lane] = val;
      if (g + gstride < groups) load_stage(g + gstride, c_lo);
      __syncthreads();
      if (ks == 0 && g < groups) {
        float t = red[wid * kWave + lane];
#pragma unroll
        for (int q = 1; q < KS; ++q) t += red[(wid + q) * kWave + lane];
        store(g, t);
      }
      __syncthreads();  // red is rewritten next round
    }
  }
}

// Split-K skinny kernel (M <= 16, K % 64 == 0): block (bx, s) owns output
// columns 16 NW bx .. +16 NW - 1 and K slice s (ksl values, a multiple of
// 64).  The block first copies the activation slice, zero-padded to 16 rows,
// into LDS (row stride 2 ksl + 16 bytes: the 16 rows of one read fall in
// distinct banks); wave w then streams weight rows 16 w .. 16 w + 15 of the
// block over the slice, lane (r, q) loading bytes 64 c + 16 q .. +15 of row
// r for chunk c, U chunks in flight, and multiplies with
// v_mfma_f32_16x16x32_bf16 (activation rows as A, weight rows as B; both
// operands put k = 64 c + 16 q + 8 h + e in k-slot 8 q + e of MFMA h).  The
// 16 x 16 partial sums go to plane s of a float32 workspace [splits, M, N];
// a second kernel adds the planes in a fixed order.  Narrow, long-K shapes
// thus keep every CU streaming while each block reads only its slice of the
// activation once.
template <int NW, int U>
__global__ __launch_bounds__(NW * 64) void fp8_skinny_splitk_kernel(const uint8_t* __restrict__ w,
                                                                    const uint16_t* __restrict__ x,
                                                                    float* __restrict__ part, int M, int64_t N,
                                                                    int64_t K, int ksl) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t slice = blockIdx.y;
  const int64_t k0 = slice * ksl;
  const int klen = int(K - k0 < ksl ? K - k0 : ksl);  // > 0, a multiple of 64
  const int row_bytes = 2 * ksl + 16;

  const int64_t n0 = int64_t(blockIdx.x) * 16 * NW + 16 * wid;
  int64_t n = n0 + r16;
  if (n >= N) n = N - 1;  // padding columns re-read the last row; never stored
  const uint8_t* wrow = w + n * K + k0 + 16 * q;
  const int nck = klen / 64;
  auto load = [&](u32x4 (&wv)[U], int c0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      wv[u] = c0 + u < nck ? ld16_stream(wrow + 64 * (c0 + u)) : u32x4{0u, 0u, 0u, 0u};
  };
  // The first weight chunks are in flight while the activation is copied.
  u32x4 wa[U], wb[U];
  load(wa, 0);

  // Activation slice: 16 rows x klen bf16 as 16-byte chunks (rows >= M are
  // zero), kBatch loads per thread in flight before their LDS stores.
  const int cpr = klen / 8;
  constexpr int kT = NW * kWave, kBatch = 8;
  for (int c0 = threadIdx.x; c0 < 16 * cpr; c0 += kT * kBatch) {
    u32x4 v[kBatch];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int c = c0 + t * kT, m = c / cpr, j = c % cpr;
      v[t] = c < 16 * cpr && m < M ? ld16(x + int64_t(m) * K + k0 + 8 * j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int c = c0 + t * kT, m = c / cpr, j = c % cpr;
      if (c < 16 * cpr) *reinterpret_cast<u32x4*>(lds + m * row_bytes + 16 * j) = v[t];
    }
  }
  __syncthreads();

  const char* xrow = lds + r16 * row_bytes + 32 * q;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nck; c0 += U) {
    if (c0 + U < nck) load(wb, c0 + U);  // next chunks in flight during this batch
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u >= nck) break;  // uniform
      const char* xa = xrow + 128 * (c0 + u);
      const v8bf a0 = *reinterpret_cast<const v8bf*>(xa);
      const v8bf a1 = *reinterpret_cast<const v8bf*>(xa + 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, e4m3x8_to_bf16x8(wa[u].x, wa[u].y), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, e4m3x8_to_bf16x8(wa[u].z, wa[u].w), acc, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) wa[u] = wb[u];
  }

  // acc[v] = D[m = 4 q + v][column n0 + r16]
  const int64_t col = n0 + r16;
  if (col < N) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * q + v;
      if (m < M) part[(slice * M + m) * N + col] = acc[v];
    }
  }
}

// Streaming matrix-core kernel for many output features (M <= 16, K in
// {1024, 2048, 3072, 4096}, aligned operands).  The weight is read the way
// the GEMV reads it -- whole contiguous row segments, non-temporal -- but by
// the DMA unit straight into LDS, and the matrix cores take their operand
// layout from there:
// * a persistent block of NW waves walks tiles of 16 weight rows; a tile is
//   KS LDS stages of 16 rows x K / KS bytes, S stages form a ring, and the
//   block keeps the next S - 1 stages in flight while it multiplies one.
//   Every DMA instruction moves 1 KiB of one row (64 lanes x 16 bytes);
//   16-byte chunk c of a stage row r sits at slot c ^ r, which the DMA
//   lanes realise by choosing which chunk each one fetches, so that the 16
//   rows of one ds_read_b128 pass fall in 16 distinct bank groups;
// * in stage h of a tile, wave w owns the K range h K / KS + [w, w + 1) K /
//   (KS NW), and it holds the activation of all its ranges (rows
//   zero-padded to 16) in registers for the whole kernel, read once;
// * per 64 K values a lane (r, q) reads 16 weight bytes of row r, widens
//   them exactly to bf16 and runs two v_mfma_f32_16x16x32_bf16 (activation
//   rows as A, weight rows as B; k = 64 c + 16 q + 8 h + e goes to k-slot
//   8 q + e of instruction h on both operands);
// * after a tile's last stage the NW partial 16 x 16 tiles meet in LDS and
//   one wave (a different one each tile) adds them in wave order and stores.
// SPLIT: K here is one slice of rows `ld` values long; block row blockIdx.y
// takes slice blockIdx.y and stores its sums, unscaled, to float32 plane
// blockIdx.y of `part` ([slices][M][N]) for the split-K reduction.
template <int NW, int SPW, int KS, int S, bool FUSED, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) void fp8_skinny_stream_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, void* __restrict__ out,
    int out_bf16, int M, int64_t N, float alpha, Epilogue epi, int64_t ld, float* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int K = 64 * NW * SPW;          // the kernel is instantiated per K (per slice with SPLIT)
  const int64_t row_len = SPLIT ? ld : int64_t(K);
  const int64_t k0 = SPLIT ? int64_t(blockIdx.y) * K : 0;
  constexpr int kRow = K / KS;              // bytes of a row in one stage
  constexpr int kSteps = SPW / KS;          // 64-value steps of a wave per stage
  constexpr int kRowParts = kRow / 1024;    // 1 KiB DMA instructions per stage row
  constexpr int kStage = 16 * kRow;
  static_assert(SPW % KS == 0 && kRow % 1024 == 0 && (16 * kRowParts) % NW == 0,
                "stages of whole KiB rows, DMA instructions split evenly over the waves");
  constexpr int kDmaPerWave = 16 * kRowParts / NW;
  static_assert((S - 1) * kDmaPerWave < 64, "wait counts fit the vmcnt field");
  v4f* red = reinterpret_cast<v4f*>(lds + S * kStage);

  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t tiles = (N + 15) / 16;
  const int64_t t0 = blockIdx.x;
  const int64_t cnt = t0 < tiles ? (tiles - 1 - t0) / gridDim.x + 1 : 0;
  if (cnt == 0) return;  // uniform: the grid never exceeds the tiles
  const int64_t stages = cnt * KS;

  // DMA of this block's stage j (tile j / KS, part j % KS) into its ring
  // slot: instruction i of wave w moves 1 KiB (part p) of stage row r.
  // A block with fewer than S stages issues only those it has (the waits
  // below count only issued stages).
  auto issue = [&](int64_t j) {
    const int64_t t = t0 + (j / KS) * gridDim.x;
    const int h = int(j % KS);
    char* slot = lds + (j % S) * kStage;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int ins = wid * kDmaPerWave + i;
      const int r = ins / kRowParts, p = ins % kRowParts;
      int64_t n = 16 * t + r;
      if (n >= N) n = N - 1;  // rows past N re-read the last row; never stored
      dma16_nt(reinterpret_cast<const char*>(w + n * row_len + k0 + h * kRow) + 16 * (64 * p + (lane ^ r)),
               slot + r * kRow + 1024 * p);
    }
  };

  issue(0);
  // Activation of this wave: xa[h][c][e] = x[r16][h K / KS + wid K / (KS NW)
  // + 64 c + 16 q + 8 e .. + 8], loaded between the first stage and the rest
  // of the prologue so that its wait does not cover the later stages.
  v8bf xa[KS][kSteps][2];
#pragma unroll
  for (int h = 0; h < KS; ++h)
#pragma unroll
    for (int c = 0; c < kSteps; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        xa[h][c][e] = r16 < M ? __builtin_bit_cast(v8bf, ld16(x + int64_t(r16) * row_len + k0 + h * kRow +
                                                                wid * (kRow / NW) + 64 * c + 16 * q + 8 * e))
                              : v8bf{};
#pragma unroll
  for (int j = 1; j < S; ++j)
    if (j < stages) issue(j);

  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int64_t j = 0; j < stages; ++j) {
    // Stage j has landed once at most `ahead` later stages' loads are pending
    // (loads complete in order).
    const int64_t ahead = stages - 1 - j < S - 1 ? stages - 1 - j : S - 1;
    if (ahead >= S - 1) wait_vm<(S - 1) * kDmaPerWave>();
    else if (ahead >= 4) wait_vm<4 * kDmaPerWave>();
    else if (ahead >= 2) wait_vm<2 * kDmaPerWave>();
    else if (ahead == 1) wait_vm<kDmaPerWave>();
    else wait_vm<0>();
    block_barrier();

    const int h = int(j % KS);
    const char* row = lds + (j % S) * kStage + r16 * kRow;
    u32x4 wv[kSteps];
#pragma unroll
    for (int c = 0; c < kSteps; ++c) {
      const int g = 4 * (wid * kSteps + c) + q;  // 16-byte chunk of the stage row
      wv[c] = *reinterpret_cast<const u32x4*>(row + 16 * (g ^ r16));
    }
#pragma unroll
    for (int hh = 0; hh < KS; ++hh) {
      if (hh != h) continue;  // uniform; keeps the register arrays statically indexed
#pragma unroll
      for (int c = 0; c < kSteps; ++c) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[hh][c][0], e4m3x8_to_bf16x8(wv[c].x, wv[c].y), acc0, 0,
                                                       0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[hh][c][1], e4m3x8_to_bf16x8(wv[c].z, wv[c].w), acc1, 0,
                                                       0, 0);
      }
    }
    const bool last = h == KS - 1;
    if (last) red[wid * kWave + lane] = acc0 + acc1;
    wait_lds();
    block_barrier();  // every wave's reads of the slot (and, at a tile's end, its partial tile) are done
    if (j + S < stages) issue(j + S);
    if (last) {
      const int64_t i = j / KS;
      if (wid == int(i % NW)) {
        v4f sum = red[lane];
#pragma unroll
        for (int v = 1; v < NW; ++v) sum += red[v * kWave + lane];
        // sum[e] = out[m = 4 q + e][n = 16 t + r16]
        const int64_t n = 16 * (t0 + i * gridDim.x) + r16;
        if (n < N) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * q + e < M) {
              if constexpr (SPLIT) part[(int64_t(blockIdx.y) * M + 4 * q + e) * N + n] = sum[e];
              else store_maybe_epi<FUSED>(out, 4 * q + e, n, N, sum[e], alpha, out_bf16, epi);
            }
        }
      }
      acc0 = v4f{0.f, 0.f, 0.f, 0.f};
      acc1 = v4f{0.f, 0.f, 0.f, 0.f};
    }
  }
}

}  // namespace

namespace {

constexpr int kMaxLds = 160 * 1024;

// fp8_skinny_kernel: a block of NWV waves per 16 G output columns.
template <int G, int U, int NWV>
hipError_t launch_skinny16(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                           int64_t K, float alpha, const Epilogue& epi, hipStream_t s) {
  if (!epi.on)
    return launch(fp8_skinny_kernel<G, U, NWV, false>, dim3((N + 16 * G - 1) / (16 * G)), dim3(NWV * kWave), 0, s, w,
                  x, out, out_bf16, int(M), N, K, alpha, epi);
  return launch(fp8_skinny_kernel<G, U, NWV, true>, dim3((N + 16 * G - 1) / (16 * G)), dim3(NWV * kWave), 0, s, w,
                x, out, out_bf16, int(M), N, K, alpha, epi);
}

// Largest activation copy (bytes) the LDS holds: 4 MG padded rows x K bf16.
int xlds_groups(int64_t M) { return M <= 4 ? 1 : (M <= 8 ? 2 : 4); }

template <int MG, int NWB, int KS, bool FUSED>
hipError_t launch_xlds_nwb(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int M, int N, int K,
                           float alpha, int num_cus, const Epilogue& epi, hipStream_t s) {
  auto kern = fp8_skinny_xlds_kernel<MG, NWB, KS, FUSED>;
  static std::atomic<uint64_t> lds_set{0};  // per instantiation, one bit per device
  if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kern), kMaxLds, lds_set)) return e;
  const int64_t lds = int64_t(K / 256) * MG * 2048 + (KS > 1 ? NWB * kWave * 4 : 0);
  const int64_t groups = (int64_t(N) + 3) / 4;
  constexpr int kGpb = NWB / KS;
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(kMaxLds / lds, 16 / NWB));
  const int64_t blocks = std::min<int64_t>((groups + kGpb - 1) / kGpb, int64_t(num_cus) * per_cu);
  return launch(kern, dim3(unsigned(blocks)), dim3(NWB * kWave), size_t(lds), s, w, x, out, out_bf16, M, N, K,
                alpha, epi);
}

template <int MG, bool FUSED>
hipError_t launch_xlds_f(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int M, int N, int K,
                       float alpha, int num_cus, const Epilogue& epi, hipStream_t s) {
  // About a dozen waves per CU in total: one large block per CU when there
  // are enough 4-row groups, otherwise smaller blocks over more CUs, and
  // with few groups the K chunks of each group split over four waves.  With
  // two m-groups the accumulators and activation operands need more than
  // the 128 registers a 16-wave block leaves each wave, so 12 (or 8) waves.
  constexpr int kBig = MG == 1 ? 16 : (MG == 2 ? 12 : 8);
  const int64_t groups = (int64_t(N) + 3) / 4;
  if (groups >= int64_t(num_cus) * kBig)
    return launch_xlds_nwb<MG, kBig, 1, FUSED>(w, x, out, out_bf16, M, N, K, alpha, num_cus, epi, s);
  if (groups >= int64_t(num_cus) * 8)
    return launch_xlds_nwb<MG, 8, 1, FUSED>(w, x, out, out_bf16, M, N, K, alpha, num_cus, epi, s);
  if (K >= 4096)
    return launch_xlds_nwb<MG, 8, 4, FUSED>(w, x, out, out_bf16, M, N, K, alpha, num_cus, epi, s);
  return launch_xlds_nwb<MG, 4, 1, FUSED>(w, x, out, out_bf16, M, N, K, alpha, num_cus, epi, s);
}

template <int MG>
hipError_t launch_xlds(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int M, int N, int K,
                       float alpha, int num_cus, const Epilogue& epi, hipStream_t s) {
  if (epi.on) return launch_xlds_f<MG, true>(w, x, out, out_bf16, M, N, K, alpha, num_cus, epi, s);
  return launch_xlds_f<MG, false>(w, x, out, out_bf16, M, N, K, alpha, num_cus, epi, s);
}

}  // namespace

// Split-K skinny GEMM: K slices of at least 256 values, enough (row block,
// slice) pairs to give every CU a block, partial planes within the
// workspace; where K is made of 2048-value slices, the streaming kernel's
// split-K form instead.  Returns hipErrorInvalidValue when the shape or
// workspace does not suit it (the caller then takes another kernel).
namespace {

constexpr int kSplitNW = 8, kSplitU = 4;

// K slices of the split-K skinny kernel for (M, N, K): slices of at most
// 4096 and at least 256 values, enough (row block, slice) pairs to cover
// the CUs.  Fills *ksl; 0 when the shape does not suit the kernel.
int64_t skinny_splits(int64_t M, int64_t N, int64_t K, int num_cus, int64_t* ksl) {
  if (M < 1 || M > 16 || K % 64 != 0) return 0;
  const int64_t row_blocks = (N + 16 * kSplitNW - 1) / (16 * kSplitNW);
  int64_t splits = (num_cus + row_blocks - 1) / row_blocks;
  splits = std::min<int64_t>(splits, K / 256);
  if (splits < 2) return 0;
  int64_t k = ((K + splits - 1) / splits + 63) / 64 * 64;
  k = std::min<int64_t>(k, 4096);
  *ksl = k;
  return (K + k - 1) / k;
}

}  // namespace

namespace {

// Slices of the streaming kernel's split-K form: 2048 values each (one slice
// instantiation), at least two; 0 when K does not split so.
constexpr int kStreamSlice = 2048;
int64_t stream_splits(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > 16 || N < 16 || N > (int64_t(1) << 31) / 16 || K % kStreamSlice != 0) return 0;
  const int64_t splits = K / kStreamSlice;
  return splits >= 2 && splits <= 65535 ? splits : 0;
}

hipError_t launch_stream_split(const uint8_t* w, const uint16_t* x, float* ws, int64_t M, int64_t N, int64_t K,
                               int num_cus, hipStream_t s);

}  // namespace

size_t fp8_skinny_splitk_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus) {
  int64_t ksl = 0;
  const int64_t splits = skinny_splits(M, N, K, num_cus, &ksl);
  if (splits < 2) return 0;  // the shape does not suit split-K
  // The call may take either split-K kernel: room for the larger plane count.
  return size_t(std::max(splits, stream_splits(M, N, K))) * size_t(M) * size_t(N) * 4;
}

hipError_t launch_fp8_skinny_splitk(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M,
                                   int64_t N, int64_t K, float alpha, int num_cus, float* ws, size_t ws_bytes,
                                   hipStream_t s, const Epilogue& epi) {
  constexpr int kNW = kSplitNW, kU = kSplitU;
  if (!ws) return hipErrorInvalidValue;
  int64_t ksl = 0;
  const int64_t splits = skinny_splits(M, N, K, num_cus, &ksl);
  if (splits < 2) return hipErrorInvalidValue;
  // Where K is made of 2048-value slices, the streaming kernel's split-K form
  // (whole weight-row segments DMA'd into LDS, activation slice in registers).
  const int64_t ssplits = stream_splits(M, N, K);
  if (ssplits > 1 && size_t(ssplits) * size_t(M) * size_t(N) * 4 <= ws_bytes &&
      reinterpret_cast<uintptr_t>(w) % 16 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0) {
    if (hipError_t e = launch_stream_split(w, x, ws, M, N, K, num_cus, s)) return e;
    return launch_splitk_reduce(ws, out, out_bf16, M, N, int(ssplits), alpha, s, epi);
  }
  const int64_t row_blocks = (N + 16 * kNW - 1) / (16 * kNW);
  if (size_t(splits) * size_t(M) * size_t(N) * 4 > ws_bytes) return hipErrorInvalidValue;
  const int lds = int(16 * (2 * ksl + 16));
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(fp8_skinny_splitk_kernel<kNW, kU>), kMaxLds,
                                     lds_set))
    return e;
  if (hipError_t e = launch(fp8_skinny_splitk_kernel<kNW, kU>, dim3(unsigned(row_blocks), unsigned(splits)),
                            dim3(kNW * kWave), size_t(lds), s, w, x, ws, int(M), N, K, int(ksl)))
    return e;
  return launch_splitk_reduce(ws, out, out_bf16, M, N, int(splits), alpha, s, epi);
}

namespace {

template <int SPW, int KS, int S, bool FUSED>
hipError_t launch_stream_k(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                           float alpha, int num_cus, const Epilogue& epi, hipStream_t s) {
  constexpr int kNW = 8;
  constexpr int K = 64 * kNW * SPW;
  constexpr int kLds = S * 16 * (K / KS) + kNW * kWave * 16;
  static_assert(kLds <= kMaxLds, "ring and partial tiles fit in LDS");
  auto kern = fp8_skinny_stream_kernel<kNW, SPW, KS, S, FUSED>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kern), kLds, lds_set)) return e;
  const int64_t tiles = (N + 15) / 16;
  const int64_t blocks = std::min<int64_t>(tiles, num_cus);
  return launch(kern, dim3(unsigned(blocks)), dim3(kNW * kWave), size_t(kLds), s, w, x, out, out_bf16, int(M), N,
                alpha, epi, int64_t(K), static_cast<float*>(nullptr));
}

template <bool FUSED>
hipError_t launch_stream(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                         int64_t K, float alpha, int num_cus, const Epilogue& epi, hipStream_t s) {
  // 128 KiB of stages in the ring (S x 16 rows x K / KS bytes).  At K = 4096
  // whole-K stages (S = 2) and half-K stages (S = 4) measured the same on
  // the 128256-row weight at M = 16 (94 us), quarter-K stages 100 us.
  switch (K) {
    case 1024: return launch_stream_k<2, 1, 8, FUSED>(w, x, out, out_bf16, M, N, alpha, num_cus, epi, s);
    case 2048: return launch_stream_k<4, 2, 8, FUSED>(w, x, out, out_bf16, M, N, alpha, num_cus, epi, s);
    case 3072: return launch_stream_k<6, 3, 8, FUSED>(w, x, out, out_bf16, M, N, alpha, num_cus, epi, s);
    case 4096: return launch_stream_k<8, 1, 2, FUSED>(w, x, out, out_bf16, M, N, alpha, num_cus, epi, s);
    default: return hipErrorInvalidValue;
  }
}

// Split-K form: grid (column blocks, K / slice); the column blocks of one
// slice share the 16-row tiles, and all blocks together fill the CUs once.
template <int SPW, int KS, int S>
hipError_t launch_stream_split_k(const uint8_t* w, const uint16_t* x, float* ws, int64_t M, int64_t N, int64_t K,
                                 int num_cus, hipStream_t s) {
  constexpr int kNW = 8;
  constexpr int kSlice = 64 * kNW * SPW;
  static_assert(kSlice == kStreamSlice, "one slice width");
  constexpr int kLds = S * 16 * (kSlice / KS) + kNW * kWave * 16;
  static_assert(kLds <= kMaxLds, "ring and partial tiles fit in LDS");
  auto kern = fp8_skinny_stream_kernel<kNW, SPW, KS, S, false, true>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kern), kLds, lds_set)) return e;
  const int64_t splits = K / kSlice;
  const int64_t tiles = (N + 15) / 16;
  const int64_t per_cu = std::max<int64_t>(1, kMaxLds / kLds);
  const int64_t bx = std::max<int64_t>(1, std::min<int64_t>(tiles, int64_t(num_cus) * per_cu / splits));
  return launch(kern, dim3(unsigned(bx), unsigned(splits)), dim3(kNW * kWave), size_t(kLds), s, w, x,
                static_cast<void*>(nullptr), 0, int(M), N, 1.f, Epilogue{}, K, ws);
}

// Whole-slice stages in a two-stage ring (72 KiB, two blocks per CU): N =
// 4096, K = 14336 at M = 4 / 8 / 16 15.0 / 15.4 / 17.8 us, against 15.8 /
// 16.3 / 18.4 with half-slice stages four deep (also two blocks per CU),
// 19.1 / 19.4 / 20.3 with eight deep (one block per CU) and 16.6 / 17.0 /
// 19.1 for the split-K skinny kernel; N = K = 14336 37.7 / 39.7 / 44.4
// against 56.9 / 57.9 / 59.4 for the latter.
hipError_t launch_stream_split(const uint8_t* w, const uint16_t* x, float* ws, int64_t M, int64_t N, int64_t K,
                               int num_cus, hipStream_t s) {
  if (stream_splits(M, N, K) < 2) return hipErrorInvalidValue;
  return launch_stream_split_k<4, 1, 2>(w, x, ws, M, N, K, num_cus, s);
}

}  // namespace

bool fp8_skinny_stream_supported(const void* w, const void* x, int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 16 && (K == 1024 || K == 2048 || K == 3072 || K == 4096) && N >= 16 &&
         N <= (int64_t(1) << 31) / 16 && reinterpret_cast<uintptr_t>(w) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(x) % 16 == 0;
}

hipError_t launch_fp8_skinny_stream(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M,
                                    int64_t N, int64_t K, float alpha, int num_cus, hipStream_t s,
                                    const Epilogue& epi) {
  if (!fp8_skinny_stream_supported(w, x, M, N, K)) return hipErrorInvalidValue;
  if (epi.on) return launch_stream<true>(w, x, out, out_bf16, M, N, K, alpha, num_cus, epi, s);
  return launch_stream<false>(w, x, out, out_bf16, M, N, K, alpha, num_cus, epi, s);
}

bool fp8_skinny_stream_wins(int64_t M, int64_t N, int64_t K) {
  if (M >= 5) return N >= 6144;
  if (M == 4) return N < 65536 && (N >= 8192 || (N >= 4096 && K == 4096));
  return M == 3 && N >= 8192 && N < 65536;
}

bool fp8_skinny_xlds_supported(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 16 && K >= 256 && K % 256 == 0 && N >= 1 && N <= (int64_t(1) << 30) &&
         int64_t(xlds_groups(M)) * K * 8 + 16 * kWave * 4 <= kMaxLds;
}

hipError_t launch_fp8_skinny(const uint8_t* w, const uint16_t* x, void* out, int out_bf16,
                             int64_t M, int64_t N, int64_t K, float alpha, int num_cus,
                             hipStream_t s, const Epilogue& epi) {
  // Many output features: the streaming kernel (whole weight rows into an
  // LDS ring).  Measured at K = 4096: M = 16, N = 128256: 94 us against 102
  // us for the 4x4x4 kernel; N = 14336: 16.6 against 19.2 us (M = 8: 15.2
  // against 18.1; M = 4: 14.7 against 15.7); N = 6144: M = 16 11.3 against
  // 14.7 us, M = 8 10.1 against 11.9; at N = 4096 (one 16-row tile per CU)
  // it loses for M >= 8 (8.8 against 8.5 us at M = 16) but wins at M = 4
  // (6.8 against 7.7 us for the GEMV, which takes M = 4 there); at M = 4 over
  // the 128256-row weight the 4x4x4 kernel keeps the lead (86 against 87-91).
  if (fp8_skinny_stream_wins(M, N, K) && fp8_skinny_stream_supported(w, x, M, N, K))
    return launch_fp8_skinny_stream(w, x, out, out_bf16, M, N, K, alpha, num_cus, s, epi);
  // Measured: for 5 <= M <= 8 the activation-in-LDS kernel wins only at
  // very many output features, where its whole-row weight bursts matter most.
  if (fp8_skinny_xlds_supported(M, N, K) && (M <= 4 || N >= 65536)) {
    switch (xlds_groups(M)) {
      case 1: return launch_xlds<1>(w, x, out, out_bf16, int(M), int(N), int(K), alpha, num_cus, epi, s);
      case 2: return launch_xlds<2>(w, x, out, out_bf16, int(M), int(N), int(K), alpha, num_cus, epi, s);
      default: return launch_xlds<4>(w, x, out, out_bf16, int(M), int(N), int(K), alpha, num_cus, epi, s);
    }
  }
  const bool wide_n = N >= 65536;
  if (M <= 4) {
    if (wide_n) {
      const int64_t blocks = (N + 63) / 64;  // 4 waves x 16 rows
      return epi.on ? launch(fp8_skinny4_kernel<4, 2, true>, dim3(blocks), dim3(256), 0, s, w, x, out, out_bf16,
                             int(M), N, K, alpha, epi)
                    : launch(fp8_skinny4_kernel<4, 2, false>, dim3(blocks), dim3(256), 0, s, w, x, out, out_bf16,
                             int(M), N, K, alpha, epi);
    }
    const int64_t blocks = (N + 15) / 16;  // 4 waves x 4 rows
    return epi.on ? launch(fp8_skinny4_kernel<1, 4, true>, dim3(blocks), dim3(256), 0, s, w, x, out, out_bf16,
                           int(M), N, K, alpha, epi)
                  : launch(fp8_skinny4_kernel<1, 4, false>, dim3(blocks), dim3(256), 0, s, w, x, out, out_bf16,
                           int(M), N, K, alpha, epi);
  }
  if (wide_n)
    return epi.on ? launch(fp8_skinny_lds_kernel<4, 512, true>, dim3((N + 63) / 64), dim3(256), 0, s, w, x, out,
                           out_bf16, int(M), N, K, alpha, epi)
                  : launch(fp8_skinny_lds_kernel<4, 512, false>, dim3((N + 63) / 64), dim3(256), 0, s, w, x, out,
                           out_bf16, int(M), N, K, alpha, epi);
  if (N >= 8192) return launch_skinny16<4, 2, 16>(w, x, out, out_bf16, M, N, K, alpha, epi, s);
  return launch_skinny16<1, 4, 16>(w, x, out, out_bf16, M, N, K, alpha, epi, s);
}

}  // namespace qlinear
