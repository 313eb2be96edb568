// LDS-tiled matrix-core GEMM with a decoded quantized weight operand:
//     out[m, n] = alpha * sum_k x[m, k] * dec(W[n, k])
// x is bfloat16 [M, K]; W is either float8_e4m3fn [N, K] (W8A16) or NVFP4
// (packed E2M1 [N, K/2] + E4M3 per-16 block scales [N, K/16], W4A16).
//
// What is computed: the "Matmul2dFp8" page (W8A16 GEMM, fp32 accumulation,
// c_type output; run_grouped for ragged MoE groups) and the "fp4_matmul"
// page (W4A16: each weight sub-tile is dequantised to bfloat16 once per
// K-strip, cooperatively by the block, into on-chip memory, and a dense bf16
// matrix multiply consumes it).  Both weight decodes are exact in bfloat16,
// so the bf16 matrix cores see exactly the decoded weight.
//
// Structure (gfx950): a 256-thread block computes a 128 x 128 output tile in
// 64-wide K strips.  Each strip, the block loads the activation tile (bf16,
// 16-byte coalesced loads) and the raw weight tile (fp8 or packed fp4 +
// scales), decodes the weight to bfloat16 while writing it to LDS, and the
// four waves (2 x 2, 64 x 64 each) run 4 x 4 v_mfma_f32_16x16x32_bf16 per
// 32-wide K step from LDS.  The next strip's global loads are issued before
// the current strip's matrix-core work, so HBM traffic overlaps compute.
// Blocks are mapped to tiles so that each XCD works on a contiguous range of
// tiles, walked in groups of 8 row tiles per column tile (L2 reuse of the
// weight tile).  This kernel serves any K and alignment and the grouped
// MoE call; K % 64 == 0 with aligned operands goes to the pipelined
// direct-to-LDS kernel of gemm_lds.hip.
#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kLdsRow = BK * 2 + 16;           // bytes per LDS row: 64 bf16 + 16 B pad
constexpr int kLdsTile = 128 * kLdsRow;        // one 128-row operand tile
constexpr int kLdsBytes = 2 * kLdsTile;        // activation tile + weight tile

// ---------------------------------------------------------------- activation tile

struct ActTile {
  const uint16_t* x;  // [M, K] bf16, row 0 of the current problem
  int64_t M, K;
  bool vec;           // K % 8 == 0 and 16-byte aligned base
};

struct ActStage { u32x4 v[4]; };

// Thread t loads chunks id = t + 256 i (i < 4): row id / 8, elements 8 (id % 8) .. +7.
__device__ __forceinline__ void act_load(const ActTile& A, int64_t m0, int64_t k0, ActStage& st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = threadIdx.x + kThreads * i;
    const int64_t m = m0 + (id >> 3);
    const int64_t k = k0 + 8 * (id & 7);
    if (m < A.M && A.vec && k + 8 <= A.K) {
      st.v[i] = ld16(A.x + m * A.K + k);
    } else {
      uint32_t e[4] = {0u, 0u, 0u, 0u};
      if (m < A.M) {
        for (int j = 0; j < 8; ++j)
          if (k + j < A.K) e[j >> 1] |= uint32_t(A.x[m * A.K + k + j]) << (16 * (j & 1));
      }
      st.v[i] = u32x4{e[0], e[1], e[2], e[3]};
    }
  }
}

__device__ __forceinline__ void act_store(char* lds, const ActStage& st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = threadIdx.x + kThreads * i;
    *reinterpret_cast<u32x4*>(lds + (id >> 3) * kLdsRow + 16 * (id & 7)) = st.v[i];
  }
}

// ---------------------------------------------------------------- FP8 weight tile

struct Fp8Tile {
  const uint8_t* w;  // [N, K] float8_e4m3fn
  int64_t N, K;
  bool vec;          // K % 16 == 0 and 16-byte aligned base
};

struct Fp8Stage { u32x4 v[2]; };

// Thread t loads chunks id = t + 256 i (i < 2): row id / 4, bytes 16 (id % 4) .. +15.
__device__ __forceinline__ void w_load(const Fp8Tile& B, int64_t n0, int64_t k0, Fp8Stage& st) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = threadIdx.x + kThreads * i;
    const int64_t n = n0 + (id >> 2);
    const int64_t k = k0 + 16 * (id & 3);
    if (n < B.N && B.vec && k + 16 <= B.K) {
      st.v[i] = ld16_stream(B.w + n * B.K + k);
    } else {
      uint32_t e[4] = {0u, 0u, 0u, 0u};
      if (n < B.N) {
        for (int j = 0; j < 16; ++j)
          if (k + j < B.K) e[j >> 2] |= uint32_t(B.w[n * B.K + k + j]) << (8 * (j & 3));
      }
      st.v[i] = u32x4{e[0], e[1], e[2], e[3]};
    }
  }
}

__device__ __forceinline__ void w_store(char* lds, const Fp8Tile&, const Fp8Stage& st) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int id = threadIdx.x + kThreads * i;
    char* dst = lds + (id >> 2) * kLdsRow + 32 * (id & 3);
    const u32x4 v = st.v[i];
    *reinterpret_cast<u32x4*>(dst) =
        u32x4{e4m3x2_to_bf16x2<false>(v.x), e4m3x2_to_bf16x2<true>(v.x),
              e4m3x2_to_bf16x2<false>(v.y), e4m3x2_to_bf16x2<true>(v.y)};
    *reinterpret_cast<u32x4*>(dst + 16) =
        u32x4{e4m3x2_to_bf16x2<false>(v.z), e4m3x2_to_bf16x2<true>(v.z),
              e4m3x2_to_bf16x2<false>(v.w), e4m3x2_to_bf16x2<true>(v.w)};
  }
}

// ---------------------------------------------------------------- NVFP4 weight tile

struct Nvfp4Tile {
  const uint8_t* packed;  // [N, K/2], even k in the low nibble
  const uint8_t* scales;  // [N, K/16] float8_e4m3fn
  int64_t N, K;           // K % 16 == 0
  bool vec;               // K % 32 == 0 and 16-byte aligned base
};

struct Nvfp4Stage { u32x4 v; float s[2]; };

// Thread t loads row t / 2, packed bytes 16 (t % 2) .. +15 (32 weights, two scale blocks).
__device__ __forceinline__ void w_load(const Nvfp4Tile& B, int64_t n0, int64_t k0, Nvfp4Stage& st) {
  const int64_t n = n0 + (threadIdx.x >> 1);
  const int64_t k = k0 + 32 * (threadIdx.x & 1);
  const int64_t row_bytes = B.K >> 1;
  if (n < B.N && B.vec && k + 32 <= B.K) {
    st.v = ld16_stream(B.packed + n * row_bytes + (k >> 1));
  } else {
    uint32_t e[4] = {0u, 0u, 0u, 0u};
    if (n < B.N) {
      for (int j = 0; j < 16; ++j)
        if (k + 2 * j < B.K) e[j >> 2] |= uint32_t(B.packed[n * row_bytes + (k >> 1) + j]) << (8 * (j & 3));
    }
    st.v = u32x4{e[0], e[1], e[2], e[3]};
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t kb = k + 16 * j;
    st.s[j] = (n < B.N && kb < B.K) ? e4m3_to_f32(B.scales[n * (B.K >> 4) + (kb >> 4)]) : 0.f;
  }
}

__device__ __forceinline__ void w_store(char* lds, const Nvfp4Tile&, const Nvfp4Stage& st) {
  char* dst = lds + (threadIdx.x >> 1) * kLdsRow + 64 * (threadIdx.x & 1);
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // dword q = bytes 4q .. 4q+3 = weights 8q .. 8q+7
    const float s = st.s[q >> 1];
    *reinterpret_cast<u32x4*>(dst + 16 * q) = u32x4{
        e2m1x2_to_bf16x2<0>(st.v[q], s), e2m1x2_to_bf16x2<1>(st.v[q], s),
        e2m1x2_to_bf16x2<2>(st.v[q], s), e2m1x2_to_bf16x2<3>(st.v[q], s)};
  }
}

// ---------------------------------------------------------------- bf16 weight tile (dense control)

// The weight tile has the activation tile's layout and loads.
struct Bf16Tile {
  const uint16_t* w;  // [N, K] bfloat16
  int64_t N, K;
  bool vec;           // K % 8 == 0 and 16-byte aligned base
};

struct Bf16Stage { ActStage a; };

__device__ __forceinline__ void w_load(const Bf16Tile& B, int64_t n0, int64_t k0, Bf16Stage& st) {
  act_load(ActTile{B.w, B.N, B.K, B.vec}, n0, k0, st.a);
}

__device__ __forceinline__ void w_store(char* lds, const Bf16Tile&, const Bf16Stage& st) { act_store(lds, st.a); }

// ---------------------------------------------------------------- one output tile

template <class T> struct StageOf;
template <> struct StageOf<Fp8Tile> { using type = Fp8Stage; };
template <> struct StageOf<Nvfp4Tile> { using type = Nvfp4Stage; };
template <> struct StageOf<Bf16Tile> { using type = Bf16Stage; };

// Expert e of a weight stack whose tile `b` addresses expert 0.
__device__ __forceinline__ Fp8Tile expert_tile(const Fp8Tile& b, int64_t e) {
  return Fp8Tile{b.w + e * b.N * b.K, b.N, b.K, b.vec};
}
__device__ __forceinline__ Nvfp4Tile expert_tile(const Nvfp4Tile& b, int64_t e) {
  return Nvfp4Tile{b.packed + e * b.N * (b.K >> 1), b.scales + e * b.N * (b.K >> 4), b.N, b.K, b.vec};
}

// Computes the 128 x 128 tile at (m0, n0) of out[M, N] (row stride N) and
// stores alpha * acc.  Every thread of the block must call it.
template <class WTile>
__device__ void gemm_tile(char* lds, const ActTile& A, const WTile& B, void* out, int out_bf16,
                          int64_t m0, int64_t n0, float alpha, const Epilogue& epi) {
  using WStage = typename StageOf<WTile>::type;
  char* lds_a = lds;
  char* lds_b = lds + kLdsTile;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int wy = wid >> 1, wx = wid & 1;
  const int r16 = lane & 15, kq = lane >> 4;

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  ActStage as;
  WStage ws;
  const int64_t nk = (A.K + BK - 1) / BK;
  act_load(A, m0, 0, as);
  w_load(B, n0, 0, ws);
  for (int64_t kt = 0; kt < nk; ++kt) {
    __syncthreads();  // previous strip's LDS reads are done
    act_store(lds_a, as);
    w_store(lds_b, B, ws);
    __syncthreads();
    if (kt + 1 < nk) {
      act_load(A, m0, (kt + 1) * BK, as);
      w_load(B, n0, (kt + 1) * BK, ws);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8bf a[4], b[4];
      const int koff = (ks * 32 + kq * 8) * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const v8bf*>(lds_a + (wy * 64 + 16 * i + r16) * kLdsRow + koff);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const v8bf*>(lds_b + (wx * 64 + 16 * j + r16) * kLdsRow + koff);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // acc[i][j][v] = C[m0 + 64 wy + 16 i + 4 kq + v][n0 + 64 wx + 16 j + r16]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + wy * 64 + 16 * i + 4 * kq + v;
      if (m >= A.M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wx * 64 + 16 * j + r16;
        if (n < B.N) store_epi(out, m, n, B.N, acc[i][j][v], alpha, out_bf16, epi);
      }
    }
}

// Block b -> (row tile, column tile).  Blocks are dealt to the 8 XCDs round
// robin, so XCD x runs blocks x, x + 8, ...; give it a contiguous range of
// tiles, and inside the range walk 8 row tiles per column tile.
__device__ __forceinline__ void tile_of_block(int64_t b, int64_t tiles_m, int64_t tiles_n,
                                              int64_t& tm, int64_t& tn) {
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

template <class WTile>
__global__ __launch_bounds__(kThreads) void gemm_dense_kernel(ActTile A, WTile B, void* __restrict__ out,
                                                              int out_bf16, float alpha, Epilogue epi) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int64_t tiles_m = (A.M + BM - 1) / BM, tiles_n = (B.N + BN - 1) / BN;
  int64_t tm, tn;
  tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
  gemm_tile(lds, A, B, out, out_bf16, tm * BM, tn * BN, alpha, epi);
}

// Ragged groups: group z = blockIdx.z covers activation rows
// a_offsets[z] .. a_offsets[z+1]-1 and uses expert expert_ids[z]; blockIdx.x is
// the column tile and row tiles of the group are taken blockIdx.y, +gridDim.y, ...
// An id outside 0..E-1 (-1 marks an inactive group) writes zeros; offsets are
// clipped to T and a group whose end does not exceed its start does nothing.
// `B` addresses expert 0 of the weight stack (FP8 or NVFP4); expert_scale
// (null: raw output) gives the factor of each expert's rows.
template <class WTile>
__global__ __launch_bounds__(kThreads) void gemm_grouped_kernel(
    const uint16_t* __restrict__ x, WTile B, const uint32_t* __restrict__ a_offsets,
    const int32_t* __restrict__ expert_ids, const float* __restrict__ expert_scale, void* __restrict__ out,
    int out_bf16, int64_t T, int64_t N, int64_t K, int64_t E, bool vec) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int64_t z = blockIdx.z;
  int64_t start = a_offsets[z], end = a_offsets[z + 1];
  start = start < T ? start : T;
  end = end < T ? end : T;
  if (end <= start) return;
  const int64_t rows = end - start;
  const int64_t e = expert_ids[z];
  const int64_t n0 = int64_t(blockIdx.x) * BN;
  for (int64_t mt = blockIdx.y; mt * BM < rows; mt += gridDim.y) {
    const int64_t m0 = mt * BM;
    if (e < 0 || e >= E) {
      for (int idx = threadIdx.x; idx < BM * BN; idx += kThreads) {
        const int64_t m = m0 + idx / BN, n = n0 + idx % BN;
        if (m < rows && n < N) store_out(out, (start + m) * N + n, 0.f, 1.f, out_bf16);
      }
      continue;
    }
    const ActTile A{x + start * K, rows, K, vec};
    gemm_tile(lds, A, expert_tile(B, e), static_cast<char*>(out) + start * N * (out_bf16 ? 2 : 4), out_bf16, m0, n0,
              expert_scale ? expert_scale[e] : 1.f, Epilogue{});
  }
}

}  // namespace

hipError_t launch_fp8_tiled(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M,
                            int64_t N, int64_t K, float alpha, int num_cus, float* ws, size_t ws_bytes,
                            hipStream_t s, const Epilogue& epi) {
  if (gemm_lds_supported(x, w, w, M, N, K))
    return launch_fp8_gemm_lds(w, x, out, out_bf16, M, N, K, alpha, num_cus, ws, ws_bytes, s, epi);
  const bool vec = (K % 16 == 0) && (reinterpret_cast<uintptr_t>(w) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  const ActTile A{x, M, K, vec};
  const Fp8Tile B{w, N, K, vec};
  const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return launch(gemm_dense_kernel<Fp8Tile>, dim3(blocks), dim3(kThreads), 0, s, A, B, out, out_bf16, alpha, epi);
}

hipError_t launch_nvfp4_tiled(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* out,
                              int out_bf16, int64_t M, int64_t N, int64_t K, float alpha, int num_cus, float* ws,
                              size_t ws_bytes, hipStream_t s, const Epilogue& epi) {
  if (gemm_lds_supported(x, packed, scales, M, N, K))
    return launch_nvfp4_gemm_lds(packed, scales, x, out, out_bf16, M, N, K, alpha, num_cus, ws, ws_bytes, s, epi);
  const bool vec = (K % 32 == 0) && (reinterpret_cast<uintptr_t>(packed) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  const ActTile A{x, M, K, vec};
  const Nvfp4Tile B{packed, scales, N, K, vec};
  const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return launch(gemm_dense_kernel<Nvfp4Tile>, dim3(blocks), dim3(kThreads), 0, s, A, B, out, out_bf16,
                alpha, epi);
}

hipError_t launch_bf16_tiled(const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                             int64_t K, float alpha, int num_cus, float* ws, size_t ws_bytes, hipStream_t s,
                             const Epilogue& epi) {
  if (bf16_lds_supported(x, w, M, N, K))
    return launch_bf16_gemm_lds(w, x, out, out_bf16, M, N, K, alpha, num_cus, ws, ws_bytes, s, epi);
  const bool vec = bf16_wide(w, x, K);
  const ActTile A{x, M, K, vec};
  const Bf16Tile B{w, N, K, vec};
  const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return launch(gemm_dense_kernel<Bf16Tile>, dim3(blocks), dim3(kThreads), 0, s, A, B, out, out_bf16, alpha, epi);
}

hipError_t launch_fp8_grouped(const uint8_t* w, const uint16_t* x, const uint32_t* a_offsets,
                              const int32_t* expert_ids, void* out, int out_bf16, int64_t G,
                              int64_t max_tokens, int64_t E, int64_t T, int64_t N, int64_t K,
                              int num_cus, hipStream_t s, const float* expert_scale) {
  if (grouped_lds_supported(x, w, G, T, N, K))
    return launch_fp8_grouped_lds(w, x, a_offsets, expert_ids, out, out_bf16, G, E, T, N, K, num_cus, s,
                                  expert_scale);
  const bool vec = (K % 16 == 0) && (reinterpret_cast<uintptr_t>(w) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  int64_t tiles_m = (max_tokens + BM - 1) / BM;
  if (tiles_m < 1) tiles_m = 1;
  if (tiles_m > 65535) tiles_m = 65535;
  (void)num_cus;
  return launch(gemm_grouped_kernel<Fp8Tile>, dim3((N + BN - 1) / BN, tiles_m, G), dim3(kThreads), 0, s, x,
                Fp8Tile{w, N, K, vec}, a_offsets, expert_ids, expert_scale, out, out_bf16, T, N, K, E, vec);
}

hipError_t launch_nvfp4_grouped(const uint8_t* packed, const uint8_t* scales, const uint16_t* x,
                                const uint32_t* a_offsets, const int32_t* expert_ids, void* out, int out_bf16,
                                int64_t G, int64_t max_tokens, int64_t E, int64_t T, int64_t N, int64_t K,
                                int num_cus, hipStream_t s, const float* expert_scale) {
  if (nvfp4_grouped_lds_supported(x, packed, scales, G, T, N, K))
    return launch_nvfp4_grouped_lds(packed, scales, x, a_offsets, expert_ids, out, out_bf16, G, E, T, N, K, num_cus,
                                    s, expert_scale);
  // The element-wise fallback: vec needs every expert's packed rows 16-byte
  // aligned (K % 32 == 0 and an aligned base).
  const bool vec = (K % 32 == 0) && (reinterpret_cast<uintptr_t>(packed) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  int64_t tiles_m = (max_tokens + BM - 1) / BM;
  if (tiles_m < 1) tiles_m = 1;
  if (tiles_m > 65535) tiles_m = 65535;
  return launch(gemm_grouped_kernel<Nvfp4Tile>, dim3((N + BN - 1) / BN, tiles_m, G), dim3(kThreads), 0, s, x,
                Nvfp4Tile{packed, scales, N, K, vec}, a_offsets, expert_ids, expert_scale, out, out_bf16, T, N, K, E,
                vec);
}

}  // namespace qlinear
