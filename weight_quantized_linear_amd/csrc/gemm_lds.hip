// Pipelined LDS GEMMs for large aligned problems:
//   * W8A16 / W4A16:  out[m, n] = alpha * sum_k x[m, k] * dec(W[n, k]),  K % 64 == 0
//     ("Matmul2dFp8" page, W8A16 GEMM; "fp4_matmul" page, W4A16 GEMM: the
//     quantized weight tile is staged on chip in its stored form and decoded
//     to bfloat16 for the matrix cores)
//   * W8A8 int8:      acc = a @ b^T (int32), out = acc * a_scale[m] * b_scale[n] + bias[n],
//     K % 64 == 0 ("int8_matmul" page)
// These are the fast paths for aligned operands; gemm_bf16.hip / int8.hip
// serve every other shape.
//
// gfx950 structure:
// * A 256-thread block (4 waves, WY along M x 4/WY along N) owns a BM x BN
//   output tile; each wave owns a (BM/WY) x (BN*WY/4) part made of 32 x 32
//   accumulator blocks for v_mfma_f32_32x32x16_bf16 / v_mfma_i32_32x32x32_i8
//   (the 32 x 32 forms sustain a higher fraction of the matrix-core peak than
//   the 16 x 16 ones).
// * K is walked in strips of 64 values through an S-stage ring of LDS
//   buffers.  Strips are fetched with global_load_lds_dwordx4 (the load unit
//   writes each lane's 16 bytes straight into LDS), up to S - 1 strips ahead
//   of the strip being multiplied, so no registers stage global data.  The
//   slot of strip s is refilled with strip s + S as soon as every wave has
//   read strip s.
// * Rows of every LDS tile are stored with their 16-byte chunks permuted:
//   chunk c of row r sits in slot c ^ swz(r), swz chosen per row length so
//   that the 16 rows one ds_read_b128 pass touches hit 16 distinct bank
//   groups.  The DMA realises the permutation by choosing which global chunk
//   each lane fetches.
// * Each strip is two steps; while the matrix cores run step s, the wave
//   already reads the operands of step s + 1 from LDS (double-buffered
//   fragment registers).  One block barrier per strip, at the step that
//   crosses into the next strip.  Scheduling hints spread the DMA issue, the
//   LDS reads and the weight decode between the MFMAs of a step: with one
//   wave per SIMD nothing else covers a stalled wave.
// * The quantized weight is decoded in registers: each lane reads the stored
//   bytes of its own operand fragment (fp8 bytes, or packed fp4 plus the
//   E4M3 block scale) and widens them to bfloat16 exactly.  Inside a strip
//   the contraction index is permuted identically on both operands so that
//   each lane's stored bytes are one contiguous chunk; the permutation does
//   not change the sum.
// * Rows past M or N are fetched from the last valid row (the DMA cannot
//   zero-fill); they only feed outputs that are not stored.  Strips past the
//   end of K are re-fetches of the last strip, so every wave issues the same
//   number of loads per strip and the wait counts stay constant.
// * Output rows are staged through LDS so that full tiles leave with 16-byte
//   stores.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

namespace {

// Blocks have NW = 4 or 8 waves (one or two per SIMD; with two, one wave's
// MFMAs cover the other's stalls); the kernels take NW as a parameter.
constexpr int kMaxLds = 160 * 1024;

__device__ __forceinline__ void dma4(const char* g, char* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds, 4, 0, 0);
}

// Raw buffer over `bytes` bytes at p (stride 0; the last dword is the
// gfx9-family raw-buffer format word).  Buffer loads address it with a
// 32-bit per-lane offset plus a uniform offset, so no 64-bit per-lane
// address registers are needed; a lane whose offset lies past the record
// count reads zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  const uint32_t n = bytes >= int64_t(0xFFFFFFFF) ? 0xFFFFFFFFu : uint32_t(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(n), 0x00020000);
}

// Buffer load of 16 (4) bytes per lane straight into LDS (lane i at lds + 16 i (4 i)).
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void bdma4(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ u32x4 lds16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }

// Slot permutation of a row with CPR 16-byte chunks (CPR in {2, 4, 8}): rows
// r and r' of one 16-row group collide in a bank group only if they also
// agree in r / (16 / CPR), which the XOR then separates.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  return (r / (16 / CPR)) & (CPR - 1);
}

// ---------------------------------------------------------------- scheduling hints

// Items of `total` given to slot m when spread evenly over slots [lo, hi).
constexpr int share(int total, int lo, int hi, int m) {
  return (m < lo || m >= hi) ? 0 : (m - lo + 1) * total / (hi - lo) - (m - lo) * total / (hi - lo);
}

template <int NM, int NV, int ND, int NA, int M>
__device__ __forceinline__ void sched_slot() {
  // Consecutive ranges of MFMA slots for the LDS reads, the VMEM loads and
  // the VALU work, in that order; absent classes take no slots.
  constexpr int parts = (ND > 0) + (NV > 0) + (NA > 0);
  constexpr int len = parts ? NM / parts : NM;
  constexpr int d_end = ND ? (NV || NA ? len : NM) : 0;
  constexpr int v_end = NV ? (NA ? d_end + len : NM) : d_end;
  constexpr int nd = share(ND, 0, d_end, M);
  constexpr int nv = share(NV, d_end, v_end, M);
  constexpr int na = share(NA, v_end, NM, M);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
  if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nd, 0);  // LDS reads
  if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, nv, 0);  // VMEM loads
  if constexpr (na > 0) __builtin_amdgcn_sched_group_barrier(0x002, na, 0);  // VALU
}

template <int NM, int NV, int ND, int NA, int... Ms>
__device__ __forceinline__ void sched_region(std::integer_sequence<int, Ms...>) {
  (sched_slot<NM, NV, ND, NA, Ms>(), ...);
}

// Order the current scheduling region as NM MFMAs with ND LDS reads spread
// over the first of them, then NV VMEM loads, then NA VALU instructions (the
// weight decode, which needs the LDS reads).
template <int NM, int NV, int ND, int NA>
__device__ __forceinline__ void interleave() {
  sched_region<NM, NV, ND, NA>(std::make_integer_sequence<int, NM>{});
}

// f(std::integral_constant<int, 0>{}) .. f(std::integral_constant<int, N - 1>{}):
// a loop whose index is a compile-time constant in the body.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------- strip DMA

// One strip of ROWS rows x SB bytes of a row-major operand (row stride `ld`
// bytes), rows r0 .. r0 + ROWS - 1 clipped to `rows`.  The strip's 16-byte
// chunks are split evenly over the waves; DMA instruction q of wave w covers
// chunks (q NW + w) kLanes .. +kLanes - 1 (row c / CPR, slot c % CPR).
template <int ROWS, int SB, int NW>
struct StripDma {
  static constexpr int kCpr = SB / 16;
  static constexpr int kChunks = ROWS * kCpr;
  static_assert(kChunks % NW == 0, "every wave issues the same number of DMA instructions");
  static constexpr int kPerWave = kChunks / NW;
  static constexpr int kLanes = kPerWave >= 64 ? 64 : kPerWave;  // active lanes per instruction
  static_assert(kPerWave % kLanes == 0, "whole instructions");
  static constexpr int kInst = kPerWave / kLanes;  // per wave per strip
  uint32_t off[kInst];
  __device__ __forceinline__ void init(int64_t r0, int64_t rows, int64_t ld) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int c = (q * NW + wid) * kLanes + (lane < kLanes ? lane : 0);
      const int r = c / kCpr;
      const int g = (c % kCpr) ^ swz<kCpr>(r);
      int64_t row = r0 + r;
      if (row >= rows) row = rows - 1;
      off[q] = uint32_t(row * ld + 16 * g);
    }
  }
  // The same without clamping, for buffer fetches: rows past `rows` lie
  // past the buffer's record count and are zero-filled.
  __device__ __forceinline__ void init_open(int64_t r0, int64_t ld) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int c = (q * NW + wid) * kLanes + (lane < kLanes ? lane : 0);
      const int r = c / kCpr;
      const int g = (c % kCpr) ^ swz<kCpr>(r);
      off[q] = uint32_t((r0 + r) * ld + 16 * g);
    }
  }
  // base = operand start + the strip's byte offset within a row (uniform)
  __device__ __forceinline__ void fetch(char* tile, const char* base) const {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kInst; ++q)
      if (kLanes == 64 || lane < kLanes) dma16(base + off[q], tile + (q * NW + wid) * kLanes * 16);
  }
  // The same through a buffer resource; soff = the strip's byte offset.
  __device__ __forceinline__ void fetch(char* tile, __amdgpu_buffer_rsrc_t rsrc, uint32_t soff) const {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kInst; ++q)
      if (kLanes == 64 || lane < kLanes) bdma16(rsrc, tile + (q * NW + wid) * kLanes * 16, off[q], soff);
  }
};

// Four bytes per row (the NVFP4 block scales of one strip); wave w fills
// rows (ROWS / NW) w .. +(ROWS / NW - 1), one dword per lane.
template <int ROWS, int NW>
struct ScaleDma {
  static constexpr int kPer = ROWS / NW;
  static_assert(kPer >= 1 && kPer <= 64 && ROWS % NW == 0, "one instruction per wave");
  static constexpr int kInst = 1;
  uint32_t off;
  __device__ __forceinline__ void init(int64_t r0, int64_t rows, int64_t ld) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int64_t row = r0 + kPer * wid + (lane < kPer ? lane : 0);
    if (row >= rows) row = rows - 1;
    off = uint32_t(row * ld);
  }
  __device__ __forceinline__ void fetch(char* tile, const char* base) const {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane < kPer) dma4(base + off, tile + kPer * wid * 4);
  }
};

// ---------------------------------------------------------------- weight policies (bf16 GEMM)
//
// A strip covers 64 values of k.  Step t in {0, 1} of a strip runs two MFMA
// k-slices e in {0, 1} of 8 values per lane; lane half h = lane / 32 holds
// values k = kmap(t, h, e) .. +7.  The activation fragment of (t, h, e) is
// the 16-byte chunk kmap / 8 of the activation row.  A policy reads the
// stored weight bytes of the wave's FN column fragments (`col0` = first
// column of the wave inside the tile) and decodes them to bfloat16.

struct Fp8Args { const uint8_t* w; };
struct Nvfp4Args { const uint8_t* packed; const uint8_t* scales; };
struct Bf16Args { const uint16_t* w; };

// fp8: 64 KM bytes per row per strip (4 KM chunks; a strip of KM = 2 is 128
// values of k, whole 128-byte lines of the weight).  Step t, half h reads
// chunk 2t + h (16 values) and feeds bytes 8e .. 8e + 7 to k-slice e.
template <int BN, int FN, int NW, int KM>
struct Fp8WeightK {
  using Args = Fp8Args;
  // Expert e of a stack [E, N, K].
  __device__ static Args expert(Args a, int64_t e, int64_t N, int64_t K) { return Args{a.w + e * N * K}; }
  static constexpr int kKM = KM;   // 64-value k blocks per strip
  static constexpr int kSB = 64 * KM;  // weight bytes per row per strip
  static constexpr int kBytes = BN * kSB;
  using Dma = StripDma<BN, kSB, NW>;
  static constexpr int kLoads = Dma::kInst;
  __device__ static constexpr int reads(int) { return FN; }  // LDS reads per step
  static constexpr int kValu = 8 * FN;                          // decode instructions per step
  __device__ static constexpr int a_chunk(int t, int h, int e) { return 2 * (2 * t + h) + e; }

  Dma dma;
  const char* w;
  uint32_t foff[2 * KM];
  u32x4 raw[FN];

  __device__ __forceinline__ void init(Args a, int64_t n0, int64_t N, int64_t K, int col0, int r, int h) {
    dma.init(n0, N, K);
    w = reinterpret_cast<const char*>(a.w);
#pragma unroll
    for (int t = 0; t < 2 * KM; ++t)
      foff[t] = uint32_t((col0 + r) * kSB + 16 * ((2 * t + h) ^ swz<4 * KM>(r)));
  }
  __device__ __forceinline__ void fetch(char* tile, int64_t strip) const { dma.fetch(tile, w + strip * kSB); }
  template <int T>
  __device__ __forceinline__ void read(const char* tile) {
#pragma unroll
    for (int j = 0; j < FN; ++j) raw[j] = lds16(tile + foff[T] + j * 32 * kSB);
  }
  template <int T>
  __device__ __forceinline__ void decode(v8bf (&b)[2][FN]) const {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      b[0][j] = e4m3x8_to_bf16x8(raw[j].x, raw[j].y);
      b[1][j] = e4m3x8_to_bf16x8(raw[j].z, raw[j].w);
    }
  }
};

template <int BN, int FN, int NW>
using Fp8Weight = Fp8WeightK<BN, FN, NW, 1>;
template <int BN, int FN, int NW>
using Fp8Weight2 = Fp8WeightK<BN, FN, NW, 2>;

// NVFP4: per row and 64-value block of k, 32 packed bytes + 4 E4M3 scale
// bytes; a strip holds KM blocks (KM = 2: 64 packed bytes, whole halves of
// 128-byte lines, and 8 scale bytes per row).  In block u of a strip, half h
// reads packed chunk 2u + h (k = 64u + 32h .. +31) once; step T = 2u + t uses
// its bytes 8t .. 8t + 7 (k = 64u + 32h + 16t .. +15, scale block 4u + 2h + t)
// and k-slice e the dword 2t + e.  The scale bytes of block u sit in a plane
// of BN dwords of their own.
template <int BN, int FN, int NW, int KM>
struct Nvfp4WeightK {
  using Args = Nvfp4Args;
  // Expert e of stacks [E, N, K/2] (packed) and [E, N, K/16] (scales).
  __device__ static Args expert(Args a, int64_t e, int64_t N, int64_t K) {
    return Args{a.packed + e * N * (K / 2), a.scales + e * N * (K / 16)};
  }
  static constexpr int kKM = KM;
  static constexpr int kPacked = BN * 32 * KM;
  static constexpr int kBytes = kPacked + BN * 4 * KM;
  using Dma = StripDma<BN, 32 * KM, NW>;
  using SDma = ScaleDma<BN, NW>;
  static constexpr int kLoads = Dma::kInst + KM * SDma::kInst;
  __device__ static constexpr int reads(int t) { return t % 2 == 0 ? 2 * FN : 0; }
  static constexpr int kValu = 34 * FN;
  __device__ static constexpr int a_chunk(int t, int h, int e) { return 8 * (t / 2) + 4 * h + 2 * (t % 2) + e; }

  Dma dma;
  SDma sdma;
  const char* packed;
  const char* scales;
  uint32_t foff[KM], soff, shift;
  u32x4 raw[FN];
  uint32_t sc[FN];

  __device__ __forceinline__ void init(Args a, int64_t n0, int64_t N, int64_t K, int col0, int r, int h) {
    dma.init(n0, N, K / 2);
    sdma.init(n0, N, K / 16);
    packed = reinterpret_cast<const char*>(a.packed);
    scales = reinterpret_cast<const char*>(a.scales);
#pragma unroll
    for (int u = 0; u < KM; ++u) foff[u] = uint32_t((col0 + r) * 32 * KM + 16 * ((2 * u + h) ^ swz<2 * KM>(r)));
    soff = uint32_t(kPacked + (col0 + r) * 4);
    shift = 16 * h;
  }
  __device__ __forceinline__ void fetch(char* tile, int64_t strip) const {
    dma.fetch(tile, packed + strip * 32 * KM);
#pragma unroll
    for (int u = 0; u < KM; ++u) sdma.fetch(tile + kPacked + u * BN * 4, scales + strip * 4 * KM + 4 * u);
  }
  template <int T>
  __device__ __forceinline__ void read(const char* tile) {
    if constexpr (T % 2 == 0) {
      constexpr int u = T / 2;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        raw[j] = lds16(tile + foff[u] + j * 32 * 32 * KM);
        sc[j] = *reinterpret_cast<const uint32_t*>(tile + soff + u * BN * 4 + j * 32 * 4);
      }
    }
  }
  template <int T>
  __device__ __forceinline__ void decode(v8bf (&b)[2][FN]) const {
    constexpr int t = T % 2;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const float s = e4m3_to_f32((sc[j] >> (shift + 8 * t)) & 0xFFu);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t d = raw[j][2 * t + e];
        const u32x4 o{e2m1x2_to_bf16x2<0>(d, s), e2m1x2_to_bf16x2<1>(d, s), e2m1x2_to_bf16x2<2>(d, s),
                      e2m1x2_to_bf16x2<3>(d, s)};
        b[e][j] = __builtin_bit_cast(v8bf, o);
      }
    }
  }
};
template <int BN, int FN, int NW>
using Nvfp4Weight = Nvfp4WeightK<BN, FN, NW, 1>;
template <int BN, int FN, int NW>
using Nvfp4Weight2 = Nvfp4WeightK<BN, FN, NW, 2>;

// Dense bf16 weight (the control): 128 bytes per row per strip, the
// activation strip's layout.  Step t, half h, k-slice e reads the chunk the
// activation fragment of (t, h, e) reads, so both operands pair the same k;
// the stored bits are the MFMA operand (no decode).
template <int BN, int FN, int NW>
struct Bf16Weight {
  using Args = Bf16Args;
  __device__ static Args expert(Args a, int64_t e, int64_t N, int64_t K) { return Args{a.w + e * N * K}; }
  static constexpr int kBytes = BN * 128;
  using Dma = StripDma<BN, 128, NW>;
  static constexpr int kLoads = Dma::kInst;
  static constexpr int kKM = 1;
  __device__ static constexpr int reads(int) { return 2 * FN; }
  static constexpr int kValu = 0;
  __device__ static constexpr int a_chunk(int t, int h, int e) { return 2 * (2 * t + h) + e; }

  Dma dma;
  const char* w;
  uint32_t foff[2][2];
  u32x4 raw[2][FN];

  __device__ __forceinline__ void init(Args a, int64_t n0, int64_t N, int64_t K, int col0, int r, int h) {
    dma.init(n0, N, 2 * K);
    w = reinterpret_cast<const char*>(a.w);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 2; ++e) foff[t][e] = uint32_t((col0 + r) * 128 + 16 * (a_chunk(t, h, e) ^ swz<8>(r)));
  }
  __device__ __forceinline__ void fetch(char* tile, int64_t strip) const { dma.fetch(tile, w + strip * 128); }
  template <int T>
  __device__ __forceinline__ void read(const char* tile) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int j = 0; j < FN; ++j) raw[e][j] = lds16(tile + foff[T][e] + j * 32 * 128);
  }
  template <int T>
  __device__ __forceinline__ void decode(v8bf (&b)[2][FN]) const {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int j = 0; j < FN; ++j) b[e][j] = __builtin_bit_cast(v8bf, raw[e][j]);
  }
};

// Block b -> (row tile, column tile).  Blocks are dealt to the 8 XCDs round
// robin, so XCD x runs blocks x, x + 8, ...; give it a contiguous range of
// tiles, and inside the range walk 8 row tiles per column tile.
__device__ __forceinline__ void tile_of_block(int64_t b, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                              int64_t& tn) {
#ifdef QLINEAR_FLAT_TILE_ORDER
  // Build option (QLINEAR_TILE_ORDER=flat in build.py) for measuring what the
  // order below buys: the plain row-major grid.
  tm = b / tiles_n;
  tn = b % tiles_n;
  return;
#endif
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

// ---------------------------------------------------------------- output staging

// OUT: 0 = float32, 1 = bfloat16 (round to nearest even; gfx950 converts in
// hardware), 2 = int32.
template <int OUT>
struct OutT {
  static constexpr int kBytes = OUT == 1 ? 2 : 4;
};

template <int OUT>
__device__ __forceinline__ void put_out(void* out, int64_t i, float v) {
  if constexpr (OUT == 1) reinterpret_cast<__bf16*>(out)[i] = static_cast<__bf16>(v);
  else reinterpret_cast<float*>(out)[i] = v;
}

// ROWS rows of a wave's output part (ROWS x 32 FN elements) staged in LDS
// so that they leave as 16-byte row segments.  Row stride: the two lane
// halves of one ds_write (rows 4 apart) hit disjoint banks.
template <int OUT, int FN, int ROWS>
struct Slab {
  static constexpr int kEs = OutT<OUT>::kBytes;
  static constexpr int kCols = 32 * FN;
  static constexpr int kStride = kEs * kCols + (kEs == 2 ? 16 : 32);
  static constexpr int kBytes = ROWS * kStride;
  static constexpr int kLanesPerRow = kCols * kEs / 16;
  static constexpr int kChunks = ROWS * kLanesPerRow;  // 16-byte pieces
  static constexpr int kInst = (kChunks + 63) / 64;
  static_assert(kLanesPerRow <= 64, "slab row layout");

  char* base;
  int lane;  // 0 .. 63
  __device__ __forceinline__ char* at(int row, int col) const { return base + row * kStride + col * kEs; }
  __device__ __forceinline__ void put_f(int row, int col, float x) const {
    if constexpr (OUT == 1) *reinterpret_cast<__bf16*>(at(row, col)) = static_cast<__bf16>(x);
    else *reinterpret_cast<float*>(at(row, col)) = x;
  }
  __device__ __forceinline__ void put_i(int row, int col, int32_t x) const {
    *reinterpret_cast<int32_t*>(at(row, col)) = x;
  }
  // Copy the slab to out rows row0 .. row0 + ROWS - 1, columns col0 ..
  // (row-major, leading dimension N elements, 16-byte aligned rows).  LDS
  // accesses of one wave complete in order, so the reads see the writes;
  // the asm barriers keep the compiler from reordering them.
  __device__ __forceinline__ void flush(void* out, int64_t N, int64_t row0, int64_t col0) const {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int idx = q * 64 + lane;
      if (kChunks % 64 == 0 || idx < kChunks) {
        const int row = idx / kLanesPerRow, cb = (idx % kLanesPerRow) * 16;
        const u32x4 d = lds16(base + row * kStride + cb);
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(out) + ((row0 + row) * N + col0) * kEs + cb) = d;
      }
    }
    asm volatile("" ::: "memory");
  }
};

// Raise the kernel's dynamic LDS limit once per kernel, then launch.
template <auto Kernel, class... Args>
hipError_t launch_big_lds(int lds_bytes, int64_t blocks, int threads, hipStream_t s, Args... args) {
  static std::atomic<uint64_t> lds_set{0};  // per kernel, one bit per device
  if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(Kernel), lds_bytes, lds_set)) return e;
  return launch(Kernel, dim3(blocks), dim3(threads), lds_bytes, s, args...);
}

int64_t tiles(int64_t M, int64_t N, int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); }

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// LDS offset of the output slabs (the int8 epilogue keeps its scales below).
constexpr int kSlabBase = 4096;

// ---------------------------------------------------------------- bf16 x quantized-weight GEMM

template <template <int, int, int> class WP, int BM, int BN, int S, int WY, int NW>
struct WqLayout {
  static constexpr int WX = NW / WY;
  static constexpr int FM = BM / WY / 32, FN = BN / WX / 32;
  using W = WP<BN, FN, NW>;
  static constexpr int kKM = W::kKM;           // 64-value k blocks per strip
  static constexpr int kAsb = 128 * kKM;       // activation bytes per row per strip
  static constexpr int kSteps = 2 * kKM;       // MFMA steps per strip
  using ADma = StripDma<BM, kAsb, NW>;
  static constexpr int kA = BM * kAsb;
  static constexpr int kStage = kA + W::kBytes;
  static constexpr int kLds = S * kStage;
  static constexpr int kLoads = ADma::kInst + W::kLoads;
  static_assert(kLds <= kMaxLds, "LDS budget");
  static_assert((S - 1) * kLoads < 64, "vmcnt range");
};

// OUT: 0 = float32, 1 = bfloat16 output.  vec: full tiles may use 16-byte
// stores (out 16-byte aligned, N * element size a multiple of 16).
// One BM x BN output tile at (m0, n0) of out[M, N] (leading dimension N).
// Strips s0 .. s0 + ns - 1 of K (64 kKM values each) are summed: all of K
// for the plain GEMM, one slice for split-K partial sums.  FUSED: the store
// applies `epi` (a separate instance, so that the epilogue's code does not
// raise the registers of the plain kernels).
template <template <int, int, int> class WP, int BM, int BN, int S, int WY, int NW, int OUT, bool FUSED = false>
__device__ __forceinline__ void wq_tile(char* lds, const uint16_t* __restrict__ x, typename WP<BN, 1, NW>::Args wa,
                                        void* __restrict__ out, int64_t M, int64_t N, int64_t K, float alpha,
                                        int vec, int64_t m0, int64_t n0, int64_t s0, int64_t ns, const Epilogue& epi) {
  using L = WqLayout<WP, BM, BN, S, WY, NW>;
  using W = typename L::W;
  constexpr int FM = L::FM, FN = L::FN;
  constexpr int kLoads = L::kLoads;  // DMA instructions per wave per strip
  constexpr int NM = 2 * FM * FN;  // MFMAs per step
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wy = wid / L::WX, wx = wid % L::WX;
  const int r = lane & 31, h = lane >> 5;
  const int row0 = wy * (BM / WY), col0 = wx * (BN / L::WX);

  // Activation rows past M are zero-filled by the buffer fetch (no traffic).
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, M * K * 2);
  typename L::ADma adma;
  adma.init_open(m0, 2 * K);
  W wq;
  wq.init(wa, n0, N, K, col0, r, h);
  constexpr int T = L::kSteps;
  uint32_t aoff[T][2];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      aoff[t][e] = uint32_t((row0 + r) * L::kAsb + 16 * (W::a_chunk(t, h, e) ^ swz<8 * L::kKM>(r)));
  const int64_t nk = ns;

  // Strip s goes to slot s % S; past the last strip it re-fetches the last one.
  auto fetch = [&](int64_t s) {
    char* st = lds + (s % S) * L::kStage;
    const int64_t src = s0 + (s < nk ? s : nk - 1);
    adma.fetch(st, rx, uint32_t(src * L::kAsb));
    wq.fetch(st + L::kA, src);
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  u32x4 aX[2][FM], aY[2][FM];
  v8bf bX[2][FN], bY[2][FN];
  auto read_a = [&](u32x4 (&a)[2][FM], const char* st, int t) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < FM; ++i) a[e][i] = lds16(st + aoff[t][e] + i * 32 * L::kAsb);
  };
  auto mma = [&](const u32x4 (&a)[2][FM], const v8bf (&b)[2][FN]) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[e][i]), b[e][j], acc[i][j],
                                                              0, 0, 0);
  };

  // A wave whose rows all lie past M (a short group or the last row tile)
  // still fetches its share of every strip and meets every barrier, but
  // reads, decodes and multiplies nothing: LIVE = false.
  auto main_loop = [&](auto live) {
    constexpr bool LIVE = decltype(live)::value;
#pragma unroll
    for (int s = 0; s < S; ++s) fetch(s);
    wait_vm<(S - 1) * kLoads>();
    block_barrier();
    if constexpr (LIVE) {
      read_a(aX, lds, 0);
      wq.template read<0>(lds + L::kA);
      wq.template decode<0>(bX);
    }

    // Steps 0 .. T - 2 of the strip at `st`: read step t + 1 while the
    // matrix cores run step t (register sets X for even t, Y for odd t).
    auto inner = [&](const char* st) {
      if constexpr (LIVE)
        static_for<T - 1>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          if constexpr (t % 2 == 0) {
            read_a(aY, st, t + 1);
            wq.template read<t + 1>(st + L::kA);
            mma(aX, bX);
            wq.template decode<t + 1>(bY);
          } else {
            read_a(aX, st, t + 1);
            wq.template read<t + 1>(st + L::kA);
            mma(aY, bY);
            wq.template decode<t + 1>(bX);
          }
          interleave<NM, 0, 2 * FM + W::reads(t + 1), W::kValu>();
        });
    };
    for (int64_t kt = 0; kt < nk - 1; ++kt) {
      inner(lds + (kt % S) * L::kStage);
      // last step: cross into strip kt + 1 (landed for every wave after the
      // barrier); slot kt % S is free once every wave's reads of it returned
      wait_lds();
      wait_vm<(S - 2) * kLoads>();
      block_barrier();
      fetch(kt + S);
      if constexpr (LIVE) {
        const char* sn = lds + ((kt + 1) % S) * L::kStage;
        read_a(aX, sn, 0);
        wq.template read<0>(sn + L::kA);
        mma(aY, bY);
        wq.template decode<0>(bX);
        interleave<NM, kLoads, 2 * FM + W::reads(0), W::kValu>();
      }
    }
    inner(lds + ((nk - 1) % S) * L::kStage);
    if constexpr (LIVE) mma(aY, bY);
    wait_vm<0>();  // no LDS write may land after the block ends
  };
  if (m0 + row0 < M) main_loop(std::true_type{});
  else main_loop(std::false_type{});

  // acc[i][j][v] = C[m0 + row0 + 32 i + 8 (v / 4) + 4 h + v % 4][n0 + col0 + 32 j + r]
  // Full tiles leave through the per-wave LDS slabs when they fit.  The
  // fused epilogue, when present, is applied to each element on its way.
  {
    auto value = [&](float a, int64_t m, int64_t n) {
      if constexpr (FUSED) return epi_apply(epi, a * alpha, m, n);
      else return a * alpha;
    };
    constexpr bool kSlabFits = kSlabBase + NW * Slab<OUT, FN, 32>::kBytes <= L::kLds;
    if (kSlabFits && vec && m0 + BM <= M && n0 + BN <= N) {
      block_barrier();  // every wave is done reading the last strip
      const Slab<OUT, FN, 32> slab{lds + kSlabBase + wid * Slab<OUT, FN, 32>::kBytes, lane};
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = 8 * (v / 4) + 4 * h + (v % 4), col = 32 * j + r;
            slab.put_f(row, col, value(acc[i][j][v], m0 + row0 + 32 * i + row, n0 + col0 + col));
          }
        slab.flush(out, N, m0 + row0 + 32 * i, n0 + col0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slab reads done before it is rewritten
      }
    } else {
      const int64_t mw = m0 + row0 + 4 * h, nw = n0 + col0 + r;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t m = mw + 32 * i + 8 * (v / 4) + (v % 4);
          if (m >= M) continue;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int64_t n = nw + 32 * j;
            if (n < N) put_out<OUT>(out, m * N + n, value(acc[i][j][v], m, n));
          }
        }
    }
  }
}

template <template <int, int, int> class WP, int BM, int BN, int S, int WY, int NW, int OUT, bool FUSED>
__global__ __launch_bounds__(64 * NW) void wq_gemm_kernel(const uint16_t* __restrict__ x,
                                                          typename WP<BN, 1, NW>::Args wa, void* __restrict__ out,
                                                          int64_t M, int64_t N, int64_t K, float alpha, int vec,
                                                          Epilogue epi) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int64_t tm, tn;
  tile_of_block(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  using L = WqLayout<WP, BM, BN, S, WY, NW>;
  wq_tile<WP, BM, BN, S, WY, NW, OUT, FUSED>(lds, x, wa, out, M, N, K, alpha, vec, tm * BM, tn * BN, 0,
                                             K / (64 * L::kKM), epi);
}

// Split-K: block b computes slice b % splits of tile b / splits into the
// float32 partial-sum plane part + slice * M * N; wq_reduce_kernel adds the
// planes.  For small M, where whole-K tiles would leave most CUs idle.
template <template <int, int, int> class WP, int BM, int BN, int S, int WY, int NW>
__global__ __launch_bounds__(64 * NW) void wq_splitk_kernel(const uint16_t* __restrict__ x,
                                                            typename WP<BN, 1, NW>::Args wa, float* __restrict__ part,
                                                            int64_t M, int64_t N, int64_t K, int splits, int vec) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int64_t slice = blockIdx.x % splits, tile = blockIdx.x / splits;
  int64_t tm, tn;
  tile_of_block(tile, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  using L = WqLayout<WP, BM, BN, S, WY, NW>;
  const int64_t nk = K / (64 * L::kKM), per = (nk + splits - 1) / splits;
  const int64_t s0 = slice * per, ns = nk - s0 < per ? nk - s0 : per;
  wq_tile<WP, BM, BN, S, WY, NW, 0>(lds, x, wa, part + slice * M * N, M, N, K, 1.f, vec, tm * BM, tn * BN, s0, ns,
                                    Epilogue{});
}

// out[i] = epilogue(alpha * sum over the planes of part[plane][i]), four
// elements per thread; element i is (i / N, i % N) of out[M, N].
template <int OUT>
__global__ __launch_bounds__(256) void wq_reduce_kernel(const float* __restrict__ part, void* __restrict__ out,
                                                        int64_t count, int splits, float alpha, int64_t N,
                                                        Epilogue epi) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  if (epi.on) {
    for (int64_t j = i; j < i + 4 && j < count; ++j) {
      float acc = part[j];
      for (int p = 1; p < splits; ++p) acc += part[p * count + j];
      put_out<OUT>(out, j, epi_apply(epi, acc * alpha, j / N, j % N));
    }
    return;
  }
  if (i + 4 <= count && count % 4 == 0) {
    // Up to eight planes' loads in flight at a time, added in plane order.
    auto plane = [&](int p) { return *reinterpret_cast<const v4f*>(part + p * count + i); };
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < splits; p0 += 8) {
      v4f t[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) t[q] = p0 + q < splits ? plane(p0 + q) : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (p0 + q >= splits) break;
        acc = p0 + q == 0 ? t[q] : acc + t[q];  // no +0 added: a -0 sum keeps its sign
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) put_out<OUT>(out, i + e, acc[e] * alpha);
  } else {
    for (int64_t j = i; j < i + 4 && j < count; ++j) {
      float acc = part[j];
      for (int p = 1; p < splits; ++p) acc += part[p * count + j];
      put_out<OUT>(out, j, acc * alpha);
    }
  }
}

// Grouped MoE W8A16 ("Matmul2dFp8" page, run_grouped): group z owns tokens
// a_offsets[z] .. a_offsets[z + 1] (clipped to T) and multiplies them by
// expert expert_ids[z]; an id outside 0 .. E - 1 writes zeros, an empty group
// writes nothing.  The work is the list of (row tile of some group, column
// tile) pairs; the block first builds the exclusive prefix sum of the
// groups' row-tile counts in LDS (after the strip ring), then walks the list,
// so only tiles that exist are launched.  The list (group-major, then row
// tile, then column tile) is cut into 8 contiguous ranges, one per XCD
// (blocks are dealt to the XCDs round robin, so block b runs on XCD b % 8);
// the XCD's blocks walk their range with a stride.  All row tiles of one
// expert then meet its weight tiles in the same L2, which each weight tile
// is fetched into once.
// WP: the weight format (Fp8Weight, or Nvfp4Weight for W4A16 experts); `wa`
// addresses expert 0 of the stack.  expert_scale (null: raw output) gives the
// factor of each expert's rows, applied before the single rounding.
template <template <int, int, int> class WP, int BM, int BN, int S, int WY, int NW, int OUT>
__global__ __launch_bounds__(64 * NW) void grouped_gemm_kernel(const uint16_t* __restrict__ x,
                                                                typename WP<BN, 1, NW>::Args wa,
                                                                const uint32_t* __restrict__ a_offsets,
                                                                const int32_t* __restrict__ expert_ids,
                                                                const float* __restrict__ expert_scale,
                                                                void* __restrict__ out, int64_t G, int64_t T,
                                                                int64_t N, int64_t K, int64_t E, int vec) {
  using L = WqLayout<WP, BM, BN, S, WY, NW>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int kEs = OutT<OUT>::kBytes;
  int* cum = reinterpret_cast<int*>(lds + L::kLds);  // cum[z] = row tiles of groups 0 .. z-1; cum[G] = total
  auto group_span = [&](int64_t z, int64_t& start, int64_t& rows) {
    int64_t b = a_offsets[z], e = a_offsets[z + 1];
    b = b < T ? b : T;
    e = e < T ? e : T;
    start = b;
    rows = e > b ? e - b : 0;
  };
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int64_t z0 = 0; z0 <= G; z0 += 64) {
      const int64_t z = z0 + lane;
      int t = 0;
      if (z < G) {
        int64_t st, rows;
        group_span(z, st, rows);
        t = int((rows + BM - 1) / BM);
      }
      int incl = t;  // inclusive prefix sum over the wave
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
      }
      if (z <= G) cum[z] = carry + incl - t;
      carry += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  const int64_t n_tiles = (N + BN - 1) / BN;
  const int64_t work = int64_t(cum[G]) * n_tiles;
  // gridDim.x is a multiple of 8: every XCD has gridDim.x / 8 blocks.
  constexpr int kXcd = 8;
  const int64_t xcd = blockIdx.x % kXcd, per_xcd = gridDim.x / kXcd;
  const int64_t lo = xcd * work / kXcd, hi = (xcd + 1) * work / kXcd;
  bool first = true;
  for (int64_t wi = lo + blockIdx.x / kXcd; wi < hi; wi += per_xcd) {
    const int mt = int(wi / n_tiles);
    const int64_t n0 = (wi % n_tiles) * BN;
    // Group of row tile mt: the last z with cum[z] <= mt (binary search).
    int64_t lo = 0, hi = G;  // cum[lo] <= mt < cum[hi]
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) / 2;
      if (cum[mid] <= mt) lo = mid;
      else hi = mid;
    }
    const int64_t z = lo;
    int64_t start, rows;
    group_span(z, start, rows);
    const int64_t m0 = int64_t(mt - cum[z]) * BM;
    const int64_t e = expert_ids[z];
    char* gout = static_cast<char*>(out) + start * N * kEs;
    if (e < 0 || e >= E) {
      for (int idx = threadIdx.x; idx < BM * BN; idx += 64 * NW) {
        const int64_t m = m0 + idx / BN, n = n0 + idx % BN;
        if (m < rows && n < N) put_out<OUT>(gout, m * N + n, 0.f);
      }
      continue;
    }
    // Tiles of one block reuse the LDS ring: wait until every wave is done
    // with the previous tile.
    if (!first) __syncthreads();
    first = false;
    wq_tile<WP, BM, BN, S, WY, NW, OUT>(lds, x + start * K, WP<BN, 1, NW>::expert(wa, e, N, K), gout, rows, N, K,
                                         expert_scale ? expert_scale[e] : 1.f, vec, m0, n0, 0, K / (64 * L::kKM),
                                         Epilogue{});
  }
}

template <template <int, int, int> class WP, int BM, int BN, int S, int WY, int NW>
hipError_t launch_wq(const uint16_t* x, typename WP<BN, 1, NW>::Args wa, void* out, int out_bf16, int64_t M,
                     int64_t N, int64_t K, float alpha, const Epilogue& epi, hipStream_t s) {
  using L = WqLayout<WP, BM, BN, S, WY, NW>;
  const int64_t blocks = tiles(M, N, BM, BN);
  const int es = out_bf16 ? 2 : 4;
  const int vec = aligned16(out) && (N * es) % 16 == 0;
  auto go = [&](auto fused) {
    constexpr bool F = decltype(fused)::value;
    if (out_bf16)
      return launch_big_lds<wq_gemm_kernel<WP, BM, BN, S, WY, NW, 1, F>>(L::kLds, blocks, 64 * NW, s, x, wa, out, M,
                                                                          N, K, alpha, vec, epi);
    return launch_big_lds<wq_gemm_kernel<WP, BM, BN, S, WY, NW, 0, F>>(L::kLds, blocks, 64 * NW, s, x, wa, out, M, N,
                                                                        K, alpha, vec, epi);
  };
  if (epi.on) return go(std::true_type{});
  return go(std::false_type{});
}

// Split-K launch: partial planes in the caller's float32 workspace.
template <template <int, int, int> class WP, int BM, int BN, int S, int WY, int NW>
hipError_t launch_wq_splitk(const uint16_t* x, typename WP<BN, 1, NW>::Args wa, void* out, int out_bf16, int64_t M,
                            int64_t N, int64_t K, float alpha, int splits, float* ws, const Epilogue& epi,
                            hipStream_t s) {
  using L = WqLayout<WP, BM, BN, S, WY, NW>;
  const int64_t blocks = tiles(M, N, BM, BN) * splits;
  const int vec = aligned16(ws) && (N * 4) % 16 == 0;
  hipError_t e = launch_big_lds<wq_splitk_kernel<WP, BM, BN, S, WY, NW>>(L::kLds, blocks, 64 * NW, s, x, wa, ws, M, N,
                                                                          K, splits, vec);
  if (e != hipSuccess) return e;
  const int64_t count = M * N, rblocks = (count + 1023) / 1024;
  if (out_bf16)
    return launch(wq_reduce_kernel<1>, dim3(rblocks), dim3(256), 0, s, ws, out, count, splits, alpha, N, epi);
  return launch(wq_reduce_kernel<0>, dim3(rblocks), dim3(256), 0, s, ws, out, count, splits, alpha, N, epi);
}

// Number of K slices for a grid of `nt` tiles whose strips hold `kv` values
// of k: enough blocks to cover the CUs, slices of at least 256 values of k,
// partial planes within the workspace.
int splitk_count(int64_t nt, int64_t M, int64_t N, int64_t K, int kv, int num_cus, size_t ws_bytes) {
  if (nt * 2 > num_cus) return 1;
  int64_t sp = num_cus / nt;
  if (sp > K / 256) sp = K / 256;
  while (sp > 1 && size_t(sp) * size_t(M) * size_t(N) * 4 > ws_bytes) --sp;
  if (sp < 2) return 1;
  const int64_t nk = K / kv;
  // The kernel gives slice i the strips i * per .. with per = ceil(nk / sp):
  // use only as many slices as that fills, so that none is empty.
  const int64_t per = (nk + sp - 1) / sp;
  sp = (nk + per - 1) / per;
  return sp < 2 ? 1 : int(sp);
}

// Partial-plane bytes of `sp` K slices of an [M, N] output (0 for whole-K).
size_t planes_bytes(int sp, int64_t M, int64_t N) { return sp > 1 ? size_t(sp) * size_t(M) * size_t(N) * 4 : 0; }

// ---------------------------------------------------------------- W8A8 int8
//
// Strips are SB bytes per row (SB / 16 chunks, SB = 64 or 128); step t of a
// strip, half h reads chunk 2t + h (k = 32t + 16h .. +15) of both operands.
// With 128-byte strips every DMA lane group covers a whole 128-byte line,
// which the L2 -> LDS path delivers at about 1.5x the rate of half lines
// (measured with 64 to 128 KiB in flight per CU: 24-26 against 32-39 bytes
// per clock per CU).
template <int BM, int BN, int S, int WY, int NW, int SB = 64>
struct I8Layout {
  static constexpr int WX = NW / WY;
  static constexpr int FM = BM / WY / 32, FN = BN / WX / 32;
  using ADma = StripDma<BM, SB, NW>;
  using BDma = StripDma<BN, SB, NW>;
  static constexpr int kA = BM * SB;
  static constexpr int kStage = kA + BN * SB;
  static constexpr int kSteps = SB / 32;  // MFMA k-steps per strip
  static constexpr int kLds = S * kStage;
  static constexpr int kLoads = ADma::kInst + BDma::kInst;
  static_assert(kLds <= kMaxLds, "LDS budget");
  static_assert((S - 1) * kLoads < 64, "vmcnt range");
  static_assert(FM >= 1 && FN >= 1 && BM % (32 * WY) == 0 && BN % (32 * WX) == 0, "wave layout");
  static_assert((BM + 2 * BN) * 4 <= kSlabBase, "epilogue scales fit");
  static_assert(kSlabBase + NW * Slab<0, FN, 32>::kBytes <= kLds, "output staging fits");
};

// OUT: 0 = float32, 1 = bfloat16 (dequantised), 2 = raw int32 accumulators.
// One BM x BN output tile at (m0, n0) of out[M, N]: a [M, K], b [N, K],
// a_scale [M], b_scale [N], bias [N] or null.  Every thread of the block
// calls it; the LDS ring starts at `lds`.
template <int BM, int BN, int S, int WY, int NW, int OUT, int SB = 64>
__device__ __forceinline__ void int8_tile(char* lds, const int8_t* __restrict__ a, const int8_t* __restrict__ b,
                                          const float* __restrict__ a_scale, const float* __restrict__ b_scale,
                                          const uint16_t* __restrict__ bias, void* __restrict__ out, int64_t M,
                                          int64_t N, int64_t K, int vec, int64_t m0, int64_t n0) {
  using L = I8Layout<BM, BN, S, WY, NW, SB>;
  constexpr int T = L::kSteps;
  static_assert(T % 2 == 0, "register sets alternate per step and a strip starts in the first");
  constexpr int FM = L::FM, FN = L::FN;
  constexpr int NM = FM * FN;  // MFMAs per step
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wy = wid / L::WX, wx = wid % L::WX;
  const int r = lane & 31, h = lane >> 5;
  const int row0 = wy * (BM / WY), col0 = wx * (BN / L::WX);

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, M * K), rb = make_rsrc(b, N * K);
  typename L::ADma adma;
  adma.init(m0, M, K);
  typename L::BDma bdma;
  bdma.init(n0, N, K);
  uint32_t aoff[T], boff[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    aoff[t] = uint32_t((row0 + r) * SB + 16 * ((2 * t + h) ^ swz<SB / 16>(r)));
    boff[t] = uint32_t(L::kA + (col0 + r) * SB + 16 * ((2 * t + h) ^ swz<SB / 16>(r)));
  }
  const int nk = int(K / SB);

  // Strip s goes to slot s % S; past the end of K it re-fetches the last
  // strip, so every wave issues kLoads loads per call.
  auto fetch = [&](int s) {
    char* st = lds + (s % S) * L::kStage;
    const int src = s < nk ? s : nk - 1;
    adma.fetch(st, ra, uint32_t(src) * SB);
    bdma.fetch(st + L::kA, rb, uint32_t(src) * SB);
  };

  // Epilogue scales of this tile, loaded before the main loop so their
  // latency hides behind it: thread t holds row m0 + t and column n0 + t.
  float pre_as = 0.f, pre_bs = 0.f, pre_bb = 0.f;
  if constexpr (OUT != 2) {
    const int t = threadIdx.x;
    if (t < BM) pre_as = a_scale[m0 + t < M ? m0 + t : M - 1];
    if (t < BN) {
      const int64_t n = n0 + t < N ? n0 + t : N - 1;
      pre_bs = b_scale[n];
      pre_bb = bias ? bf16_to_f32(bias[n]) : 0.f;
    }
  }

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};

  u32x4 aX[FM], bX[FN], aY[FM], bY[FN];
  auto read = [&](u32x4 (&fa)[FM], u32x4 (&fb)[FN], const char* st, int t) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = lds16(st + aoff[t] + i * 32 * SB);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = lds16(st + boff[t] + j * 32 * SB);
  };
  auto mma = [&](const u32x4 (&fa)[FM], const u32x4 (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, fa[i]), __builtin_bit_cast(v4i, fb[j]),
                                                          acc[i][j], 0, 0, 0);
  };

#pragma unroll
  for (int s = 0; s < S; ++s) fetch(s);
  wait_vm<(S - 1) * L::kLoads>();
  block_barrier();
  read(aX, bX, lds, 0);

  // Steps 0 .. T - 2 of the strip in slot `st`: read step t + 1 while the
  // matrix cores run step t (register sets X for even t, Y for odd t).
  auto inner = [&](const char* st) {
#pragma unroll
    for (int t = 0; t + 1 < T; ++t) {
      if (t % 2 == 0) {
        read(aY, bY, st, t + 1);
        mma(aX, bX);
      } else {
        read(aX, bX, st, t + 1);
        mma(aY, bY);
      }
      interleave<NM, 0, FM + FN, 0>();
    }
  };
  for (int kt = 0; kt < nk - 1; ++kt) {
    inner(lds + (kt % S) * L::kStage);
    // Cross into strip kt + 1 (landed for every wave after the barrier); the
    // slot of strip kt is free once every wave's reads of it have returned.
    wait_lds();
    wait_vm<(S - 2) * L::kLoads>();
    block_barrier();
    fetch(kt + S);
    read(aX, bX, lds + ((kt + 1) % S) * L::kStage, 0);
    mma(aY, bY);
    interleave<NM, L::kLoads, FM + FN, 0>();
  }
  inner(lds + ((nk - 1) % S) * L::kStage);
  mma(aY, bY);
  wait_vm<0>();  // no LDS write may land after the block ends

  // Scales through LDS (free now): as[BM], bs[BN], bb[BN].
  float* sh_as = reinterpret_cast<float*>(lds);
  float* sh_bs = sh_as + BM;
  float* sh_bb = sh_bs + BN;
  block_barrier();  // every wave is done reading the last strip
  if constexpr (OUT != 2) {
    const int t = threadIdx.x;
    if (t < BM) sh_as[t] = pre_as;
    if (t < BN) {
      sh_bs[t] = pre_bs;
      sh_bb[t] = pre_bb;
    }
    __syncthreads();
  }
  float bs[FN], bb[FN];
  if constexpr (OUT != 2) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      bs[j] = sh_bs[col0 + r + 32 * j];
      bb[j] = sh_bb[col0 + r + 32 * j];
    }
  }
  // Element (i, j, v): row m0 + row0 + 32 i + 8 (v / 4) + 4 h + v % 4, column n0 + col0 + 32 j + r.
  auto value = [&](int i, int j, int v, const v4f& as4) {
    return float(acc[i][j][v]) * as4[v % 4] * bs[j] + bb[j];
  };
  auto scales4 = [&](int i, int q) {  // a_scale of rows 32 i + 8 q + 4 h .. +3 of the wave part
    v4f t{};
    if constexpr (OUT != 2) t = *reinterpret_cast<const v4f*>(sh_as + row0 + 32 * i + 8 * q + 4 * h);
    return t;
  };

  if (vec && m0 + BM <= M && n0 + BN <= N) {
    const Slab<OUT, FN, 32> slab{lds + kSlabBase + wid * Slab<OUT, FN, 32>::kBytes, lane};
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f as4 = scales4(i, q);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int row = 8 * q + 4 * h + p, col = 32 * j + r;
            if constexpr (OUT == 2) slab.put_i(row, col, acc[i][j][4 * q + p]);
            else slab.put_f(row, col, value(i, j, 4 * q + p, as4));
          }
      }
      slab.flush(out, N, m0 + row0 + 32 * i, n0 + col0);
      wait_lds();  // slab reads done before it is rewritten
    }
  } else {
    const int64_t mw = m0 + row0 + 4 * h, nw = n0 + col0 + r;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f as4 = scales4(i, q);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int64_t m = mw + 32 * i + 8 * q + p;
          if (m >= M) continue;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int64_t n = nw + 32 * j;
            if (n >= N) continue;
            if constexpr (OUT == 2) reinterpret_cast<int32_t*>(out)[m * N + n] = acc[i][j][4 * q + p];
            else put_out<OUT>(out, m * N + n, value(i, j, 4 * q + p, as4));
          }
        }
      }
  }
}

template <int BM, int BN, int S, int WY, int NW, int OUT, int SB>
__global__ __launch_bounds__(64 * NW) void int8_gemm_lds_kernel(const int8_t* __restrict__ a,
                                                                 const int8_t* __restrict__ b,
                                                                 const float* __restrict__ a_scale,
                                                                 const float* __restrict__ b_scale,
                                                                 const uint16_t* __restrict__ bias,
                                                                 void* __restrict__ out, int64_t M, int64_t N,
                                                                 int64_t K, int vec) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int64_t tm, tn;
  tile_of_block(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  int8_tile<BM, BN, S, WY, NW, OUT, SB>(lds, a, b, a_scale, b_scale, bias, out, M, N, K, vec, tm * BM, tn * BN);
}

// Grouped MoE W8A8: the ragged walk of grouped_gemm_kernel (prefix sum of
// the groups' row tiles in LDS after the strip ring, one contiguous range
// of (row tile, column tile) pairs per XCD) over int8 tiles.  Group z uses
// rows a_offsets[z] .. (clipped to T) of a / a_scale and expert
// e = expert_ids[z] of b [E, N, K], b_scale [E, N] and bias [E, N]; an id
// outside 0 .. E - 1 writes zeros.
template <int BM, int BN, int S, int WY, int NW, int OUT, int SB = 64>
__global__ __launch_bounds__(64 * NW) void int8_grouped_kernel(
    const int8_t* __restrict__ a, const int8_t* __restrict__ b, const float* __restrict__ a_scale,
    const float* __restrict__ b_scale, const uint16_t* __restrict__ bias, const uint32_t* __restrict__ a_offsets,
    const int32_t* __restrict__ expert_ids, void* __restrict__ out, int64_t G, int64_t T, int64_t N, int64_t K,
    int64_t E, int vec) {
  using L = I8Layout<BM, BN, S, WY, NW, SB>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int kEs = OUT == 1 ? 2 : 4;
  int* cum = reinterpret_cast<int*>(lds + L::kLds);  // cum[z] = row tiles of groups 0 .. z-1; cum[G] = total
  auto group_span = [&](int64_t z, int64_t& start, int64_t& rows) {
    int64_t lo = a_offsets[z], hi = a_offsets[z + 1];
    lo = lo < T ? lo : T;
    hi = hi < T ? hi : T;
    start = lo;
    rows = hi > lo ? hi - lo : 0;
  };
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int64_t z0 = 0; z0 <= G; z0 += 64) {
      const int64_t z = z0 + lane;
      int t = 0;
      if (z < G) {
        int64_t st, rows;
        group_span(z, st, rows);
        t = int((rows + BM - 1) / BM);
      }
      int incl = t;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
      }
      if (z <= G) cum[z] = carry + incl - t;
      carry += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  const int64_t n_tiles = (N + BN - 1) / BN;
  const int64_t work = int64_t(cum[G]) * n_tiles;
  constexpr int kXcd = 8;  // gridDim.x is a multiple of 8
  const int64_t xcd = blockIdx.x % kXcd, per_xcd = gridDim.x / kXcd;
  const int64_t w_lo = xcd * work / kXcd, w_hi = (xcd + 1) * work / kXcd;
  bool first = true;
  for (int64_t wi = w_lo + blockIdx.x / kXcd; wi < w_hi; wi += per_xcd) {
    const int mt = int(wi / n_tiles);
    const int64_t n0 = (wi % n_tiles) * BN;
    int64_t lo = 0, hi = G;  // cum[lo] <= mt < cum[hi]
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) / 2;
      if (cum[mid] <= mt) lo = mid;
      else hi = mid;
    }
    const int64_t z = lo;
    int64_t start, rows;
    group_span(z, start, rows);
    const int64_t m0 = int64_t(mt - cum[z]) * BM;
    const int64_t e = expert_ids[z];
    char* gout = static_cast<char*>(out) + start * N * kEs;
    if (e < 0 || e >= E) {
      for (int idx = threadIdx.x; idx < BM * BN; idx += 64 * NW) {
        const int64_t m = m0 + idx / BN, n = n0 + idx % BN;
        if (m < rows && n < N) {
          if constexpr (OUT == 2) reinterpret_cast<int32_t*>(gout)[m * N + n] = 0;
          else put_out<OUT>(gout, m * N + n, 0.f);
        }
      }
      continue;
    }
    if (!first) __syncthreads();  // the previous tile's LDS use is over for every wave
    first = false;
    int8_tile<BM, BN, S, WY, NW, OUT, SB>(lds, a + start * K, b + e * N * K, a_scale ? a_scale + start : nullptr,
                                      b_scale ? b_scale + e * N : nullptr,
                                      bias ? bias + e * N : nullptr, gout, rows, N, K, vec, m0, n0);
  }
}

// ---------------------------------------------------------------- FP8 W8A8
//
// fp8 x fp8 -> float32 on v_mfma_scale_f32_32x32x64_f8f6f4 (both operands
// E4M3, block scales 2^0): the operands have the int8 kernel's byte layout,
// strips and DMA.  One instruction consumes a whole 64-byte strip: lane
// (r, h) supplies the two 16-byte chunks the int8 kernel reads in its two
// steps (chunks h and 2 + h of the row), for both operands alike, so A and
// B pair the same k in every slot.  The fragments of strip s + 1 are read
// while the matrix cores run strip s (two register sets, loop unrolled by
// two); one block barrier per strip.  out = alpha * acc (alpha = input_scale
// * weight_scale), one rounding.
template <int BM, int BN, int S, int WY, int NW, int OUT>
__global__ __launch_bounds__(64 * NW) void fp8_w8a8_lds_kernel(const uint8_t* __restrict__ a,
                                                                const uint8_t* __restrict__ b,
                                                                void* __restrict__ out, int64_t M, int64_t N,
                                                                int64_t K, float alpha, int vec) {
  using L = I8Layout<BM, BN, S, WY, NW>;
  constexpr int FM = L::FM, FN = L::FN;
  constexpr int NM = FM * FN;  // MFMAs per strip
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int64_t tm, tn;
  tile_of_block(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wy = wid / L::WX, wx = wid % L::WX;
  const int r = lane & 31, h = lane >> 5;
  const int row0 = wy * (BM / WY), col0 = wx * (BN / L::WX);

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, M * K), rb = make_rsrc(b, N * K);
  typename L::ADma adma;
  adma.init(m0, M, K);
  typename L::BDma bdma;
  bdma.init(n0, N, K);
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    aoff[t] = uint32_t((row0 + r) * 64 + 16 * ((2 * t + h) ^ swz<4>(r)));
    boff[t] = uint32_t(L::kA + (col0 + r) * 64 + 16 * ((2 * t + h) ^ swz<4>(r)));
  }
  const int nk = int(K / 64);

  auto fetch = [&](int s) {
    char* st = lds + (s % S) * L::kStage;
    const int src = s < nk ? s : nk - 1;
    adma.fetch(st, ra, uint32_t(src) * 64);
    bdma.fetch(st + L::kA, rb, uint32_t(src) * 64);
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  // Fragment of a strip: 32 bytes per lane, elements 0..3 = the chunk of
  // step 0, elements 4..7 = the chunk of step 1.
  v8i aP[FM], bP[FN], aQ[FM], bQ[FN];
  auto read = [&](v8i (&fa)[FM], v8i (&fb)[FN], const char* st) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      fa[i].lo = __builtin_bit_cast(v4i, lds16(st + aoff[0] + i * 32 * 64));
      fa[i].hi = __builtin_bit_cast(v4i, lds16(st + aoff[1] + i * 32 * 64));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      fb[j].lo = __builtin_bit_cast(v4i, lds16(st + boff[0] + j * 32 * 64));
      fb[j].hi = __builtin_bit_cast(v4i, lds16(st + boff[1] + j * 32 * 64));
    }
  };
  auto mma = [&](const v8i (&fa)[FM], const v8i (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 127, 0, 127);
  };
  // Strip kt + 1 has landed for every wave after the barrier; the slot of
  // strip kt is free once every wave's reads of it have returned.
  auto cross = [&](int kt) {
    wait_lds();
    wait_vm<(S - 2) * L::kLoads>();
    block_barrier();
    fetch(kt + S);
  };

#pragma unroll
  for (int s = 0; s < S; ++s) fetch(s);
  wait_vm<(S - 1) * L::kLoads>();
  block_barrier();
  read(aP, bP, lds);
  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    cross(kt);
    read(aQ, bQ, lds + ((kt + 1) % S) * L::kStage);
    mma(aP, bP);
    interleave<NM, L::kLoads, 2 * (FM + FN), 0>();
    cross(kt + 1);
    read(aP, bP, lds + ((kt + 2) % S) * L::kStage);
    mma(aQ, bQ);
    interleave<NM, L::kLoads, 2 * (FM + FN), 0>();
  }
  if (kt + 1 < nk) {  // two strips left: kt (in P) and kt + 1
    cross(kt);
    read(aQ, bQ, lds + ((kt + 1) % S) * L::kStage);
    mma(aP, bP);
    wait_lds();
    mma(aQ, bQ);
  } else {            // one strip left: kt (in P)
    mma(aP, bP);
  }
  wait_vm<0>();  // no LDS write may land after the block ends

  // acc[i][j][v] = C[m0 + row0 + 32 i + 8 (v / 4) + 4 h + v % 4][n0 + col0 + 32 j + r]
  constexpr bool kSlabFits = kSlabBase + NW * Slab<OUT, FN, 32>::kBytes <= L::kLds;
  if (kSlabFits && vec && m0 + BM <= M && n0 + BN <= N) {
    block_barrier();  // every wave is done reading the last strip
    const Slab<OUT, FN, 32> slab{lds + kSlabBase + wid * Slab<OUT, FN, 32>::kBytes, lane};
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) slab.put_f(8 * (v / 4) + 4 * h + (v % 4), 32 * j + r, acc[i][j][v] * alpha);
      slab.flush(out, N, m0 + row0 + 32 * i, n0 + col0);
      wait_lds();  // slab reads done before it is rewritten
    }
  } else {
    const int64_t mw = m0 + row0 + 4 * h, nw = n0 + col0 + r;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = mw + 32 * i + 8 * (v / 4) + (v % 4);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t n = nw + 32 * j;
          if (n < N) put_out<OUT>(out, m * N + n, acc[i][j][v] * alpha);
        }
      }
  }
}

// The same GEMM with the A fragments refreshed in place: the fragments of
// A row block i for strip s + 1 are read right after the MFMAs of block i
// for strip s, so only one set of A fragments (and two of B) is live.  This
// fits a 256 x 256 tile (128 x 64 per wave) in the 256 registers a wave has
// at two waves per SIMD.  Strips of SB = 64 or 128 bytes per row: a 128-byte
// strip is two 64-value k-steps, with one barrier and one DMA round per strip.
template <int BM, int BN, int S, int WY, int NW, int OUT, int SB = 64>
__global__ __launch_bounds__(64 * NW) void fp8_w8a8_lds2_kernel(const uint8_t* __restrict__ a,
                                                                 const uint8_t* __restrict__ b,
                                                                 void* __restrict__ out, int64_t M, int64_t N,
                                                                 int64_t K, float alpha, int vec) {
  using L = I8Layout<BM, BN, S, WY, NW, SB>;
  constexpr int FM = L::FM, FN = L::FN;
  constexpr int U = SB / 64;  // k-steps of 64 values per strip
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int64_t tm, tn;
  tile_of_block(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wy = wid / L::WX, wx = wid % L::WX;
  const int r = lane & 31, h = lane >> 5;
  const int row0 = wy * (BM / WY), col0 = wx * (BN / L::WX);

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, M * K), rb = make_rsrc(b, N * K);
  typename L::ADma adma;
  adma.init(m0, M, K);
  typename L::BDma bdma;
  bdma.init(n0, N, K);
  // k-step u of a strip: lane half h supplies chunks 4u + h and 4u + 2 + h
  uint32_t aoff[U][2], boff[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      aoff[u][e] = uint32_t((row0 + r) * SB + 16 * ((4 * u + 2 * e + h) ^ swz<SB / 16>(r)));
      boff[u][e] = uint32_t(L::kA + (col0 + r) * SB + 16 * ((4 * u + 2 * e + h) ^ swz<SB / 16>(r)));
    }
  const int nk = int(K / SB);

  auto fetch = [&](int s) {
    char* st = lds + (s % S) * L::kStage;
    const int src = s < nk ? s : nk - 1;
    adma.fetch(st, ra, uint32_t(src) * SB);
    bdma.fetch(st + L::kA, rb, uint32_t(src) * SB);
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  v8i fa[FM], bP[FN], bQ[FN];
  auto read_a = [&](int i, const char* st, int u) {
    fa[i].lo = __builtin_bit_cast(v4i, lds16(st + aoff[u][0] + i * 32 * SB));
    fa[i].hi = __builtin_bit_cast(v4i, lds16(st + aoff[u][1] + i * 32 * SB));
  };
  auto read_b = [&](v8i (&fb)[FN], const char* st, int u) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      fb[j].lo = __builtin_bit_cast(v4i, lds16(st + boff[u][0] + j * 32 * SB));
      fb[j].hi = __builtin_bit_cast(v4i, lds16(st + boff[u][1] + j * 32 * SB));
    }
  };
  // MFMAs of the current k-step (A in fa, B in fb) while the fragments of
  // the next one (k-step u of the strip at `next`) are read: B first, then A
  // block by block behind the MFMAs that last use it.  `last` multiplies the
  // final k-step.
  auto step = [&](const v8i (&fb)[FN], v8i (&fb_next)[FN], const char* next, int u) {
    read_b(fb_next, next, u);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 127, 0, 127);
      read_a(i, next, u);
    }
  };
  auto last = [&](const v8i (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 127, 0, 127);
  };
  auto order = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x020, L::kLoads, 0);  // DMA issue
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * FN, 0);     // B reads
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);  // block i's MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // then its A reads
    }
  };
  // With two stages the strip fetched at a crossing has one strip's time to
  // land: its B half (the weight, usually from HBM) goes out right after the
  // barrier and its A half one k-step later, which spreads the DMA issue
  // (4096 x 12288 x 3072: 131-133 -> 127.5-129.5 us; the same split gained
  // nothing in the int8 kernel, which keeps one fetch).
  auto fetch_a = [&](int s) {
    adma.fetch(lds + (s % S) * L::kStage, ra, uint32_t(s < nk ? s : nk - 1) * SB);
  };
  auto fetch_b = [&](int s) {
    bdma.fetch(lds + (s % S) * L::kStage + L::kA, rb, uint32_t(s < nk ? s : nk - 1) * SB);
  };
  constexpr bool kSplit = S == 2 && U > 1;
  auto cross = [&](int kt) {
    wait_lds();
    wait_vm<(S - 2) * L::kLoads>();
    block_barrier();
    if constexpr (kSplit) fetch_b(kt + S);
    else fetch(kt + S);
  };

#pragma unroll
  for (int s = 0; s < S; ++s) fetch(s);
  wait_vm<(S - 1) * L::kLoads>();
  block_barrier();
#pragma unroll
  for (int i = 0; i < FM; ++i) read_a(i, lds, 0);
  read_b(bP, lds, 0);
  auto advance = [&](const char* next, int u) {  // into k-step u of the strip at `next`
    step(bP, bQ, next, u);
    order();
#pragma unroll
    for (int j = 0; j < FN; ++j) bP[j] = bQ[j];
  };
  for (int kt = 0; kt + 1 < nk; ++kt) {
    if constexpr (kSplit)
      if (kt >= 1) fetch_a(kt - 1 + S);  // its slot was freed at the last crossing
#pragma unroll
    for (int u = 1; u < U; ++u) advance(lds + (kt % S) * L::kStage, u);
    cross(kt);
    advance(lds + ((kt + 1) % S) * L::kStage, 0);
  }
#pragma unroll
  for (int u = 1; u < U; ++u) advance(lds + ((nk - 1) % S) * L::kStage, u);
  wait_lds();
  last(bP);
  wait_vm<0>();  // no LDS write may land after the block ends

  // acc[i][j][v] = C[m0 + row0 + 32 i + 8 (v / 4) + 4 h + v % 4][n0 + col0 + 32 j + r]
  constexpr bool kSlabFits = kSlabBase + NW * Slab<OUT, FN, 32>::kBytes <= L::kLds;
  if (kSlabFits && vec && m0 + BM <= M && n0 + BN <= N) {
    block_barrier();  // every wave is done reading the last strip
    const Slab<OUT, FN, 32> slab{lds + kSlabBase + wid * Slab<OUT, FN, 32>::kBytes, lane};
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) slab.put_f(8 * (v / 4) + 4 * h + (v % 4), 32 * j + r, acc[i][j][v] * alpha);
      slab.flush(out, N, m0 + row0 + 32 * i, n0 + col0);
      wait_lds();  // slab reads done before it is rewritten
    }
  } else {
    const int64_t mw = m0 + row0 + 4 * h, nw = n0 + col0 + r;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = mw + 32 * i + 8 * (v / 4) + (v % 4);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t n = nw + 32 * j;
          if (n < N) put_out<OUT>(out, m * N + n, acc[i][j][v] * alpha);
        }
      }
  }
}

// The W8A8 int8 GEMM with the structure of fp8_w8a8_lds2_kernel: k-steps of
// 64 values whose fragments hold chunks h and 2 + h of the step (lane half
// h), each pair multiplied by two v_mfma_i32_32x32x32_i8 (the low halves:
// k = 0 .. 31 of the step, the high halves: 32 .. 63), the A fragments
// refreshed in place behind the MFMAs that last use them, and the int8
// kernel's dequant epilogue (acc * a_scale[m] * b_scale[n] + bias[n]).
template <int BM, int BN, int S, int WY, int NW, int OUT, int SB = 64>
__global__ __launch_bounds__(64 * NW) void int8_lds2_kernel(const int8_t* __restrict__ a,
                                                             const int8_t* __restrict__ b,
                                                             const float* __restrict__ a_scale,
                                                             const float* __restrict__ b_scale,
                                                             const uint16_t* __restrict__ bias,
                                                             void* __restrict__ out, int64_t M, int64_t N,
                                                             int64_t K, int vec) {
  using L = I8Layout<BM, BN, S, WY, NW, SB>;
  constexpr int FM = L::FM, FN = L::FN;
  constexpr int U = SB / 64;  // k-steps of 64 values per strip
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int64_t tm, tn;
  tile_of_block(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wy = wid / L::WX, wx = wid % L::WX;
  const int r = lane & 31, h = lane >> 5;
  const int row0 = wy * (BM / WY), col0 = wx * (BN / L::WX);

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, M * K), rb = make_rsrc(b, N * K);
  typename L::ADma adma;
  adma.init(m0, M, K);
  typename L::BDma bdma;
  bdma.init(n0, N, K);
  // k-step u of a strip: lane half h supplies chunks 4u + h and 4u + 2 + h
  uint32_t aoff[U][2], boff[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      aoff[u][e] = uint32_t((row0 + r) * SB + 16 * ((4 * u + 2 * e + h) ^ swz<SB / 16>(r)));
      boff[u][e] = uint32_t(L::kA + (col0 + r) * SB + 16 * ((4 * u + 2 * e + h) ^ swz<SB / 16>(r)));
    }
  const int nk = int(K / SB);

  auto fetch = [&](int s) {
    char* st = lds + (s % S) * L::kStage;
    const int src = s < nk ? s : nk - 1;
    adma.fetch(st, ra, uint32_t(src) * SB);
    bdma.fetch(st + L::kA, rb, uint32_t(src) * SB);
  };

  // Epilogue scales of this tile, loaded before the main loop so their
  // latency hides behind it: thread t holds row m0 + t and column n0 + t.
  float pre_as = 0.f, pre_bs = 0.f, pre_bb = 0.f;
  if constexpr (OUT != 2) {
    const int t = threadIdx.x;
    if (t < BM) pre_as = a_scale[m0 + t < M ? m0 + t : M - 1];
    if (t < BN) {
      const int64_t n = n0 + t < N ? n0 + t : N - 1;
      pre_bs = b_scale[n];
      pre_bb = bias ? bf16_to_f32(bias[n]) : 0.f;
    }
  }

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};

  v8i fa[FM], bP[FN], bQ[FN];
  auto read_a = [&](int i, const char* st, int u) {
    fa[i].lo = __builtin_bit_cast(v4i, lds16(st + aoff[u][0] + i * 32 * SB));
    fa[i].hi = __builtin_bit_cast(v4i, lds16(st + aoff[u][1] + i * 32 * SB));
  };
  auto read_b = [&](v8i (&fb)[FN], const char* st, int u) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      fb[j].lo = __builtin_bit_cast(v4i, lds16(st + boff[u][0] + j * 32 * SB));
      fb[j].hi = __builtin_bit_cast(v4i, lds16(st + boff[u][1] + j * 32 * SB));
    }
  };
  // MFMAs of the current k-step (A in fa, B in fb) while the fragments of
  // the next one (k-step u of the strip at `next`) are read: B first, then A
  // block by block behind the MFMAs that last use it.  `last` multiplies the
  // final k-step.
  auto step = [&](const v8i (&fb)[FN], v8i (&fb_next)[FN], const char* next, int u) {
    read_b(fb_next, next, u);
    // low halves of every block first, so that the two MFMAs into one
    // accumulator are FM * FN instructions apart
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i].lo, fb[j].lo, acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i].hi, fb[j].hi, acc[i][j], 0, 0, 0);
      read_a(i, next, u);
    }
  };
  auto last = [&](const v8i (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i].lo, fb[j].lo, acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i].hi, fb[j].hi, acc[i][j], 0, 0, 0);
  };
  auto order = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x020, L::kLoads, 0);  // DMA issue
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * FN, 0);     // B reads
    __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);    // the low halves
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);  // block i's high halves
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // then its A reads
    }
  };
  // With two stages the strip fetched at a crossing has one strip's time to
  // land: its B half (the weight, usually from HBM) goes out right after the
  // barrier and its A half one k-step later, which spreads the DMA issue
  // (4096 x 12288 x 3072: 131-133 -> 127.5-129.5 us; the same split gained
  // nothing in the int8 kernel, which keeps one fetch).
  auto fetch_a = [&](int s) {
    adma.fetch(lds + (s % S) * L::kStage, ra, uint32_t(s < nk ? s : nk - 1) * SB);
  };
  auto fetch_b = [&](int s) {
    bdma.fetch(lds + (s % S) * L::kStage + L::kA, rb, uint32_t(s < nk ? s : nk - 1) * SB);
  };
  constexpr bool kSplit = S == 2 && U > 1;
  auto cross = [&](int kt) {
    wait_lds();
    wait_vm<(S - 2) * L::kLoads>();
    block_barrier();
    if constexpr (kSplit) fetch_b(kt + S);
    else fetch(kt + S);
  };

#pragma unroll
  for (int s = 0; s < S; ++s) fetch(s);
  wait_vm<(S - 1) * L::kLoads>();
  block_barrier();
#pragma unroll
  for (int i = 0; i < FM; ++i) read_a(i, lds, 0);
  read_b(bP, lds, 0);
  auto advance = [&](const char* next, int u) {  // into k-step u of the strip at `next`
    step(bP, bQ, next, u);
    order();
#pragma unroll
    for (int j = 0; j < FN; ++j) bP[j] = bQ[j];
  };
  for (int kt = 0; kt + 1 < nk; ++kt) {
    if constexpr (kSplit)
      if (kt >= 1) fetch_a(kt - 1 + S);  // its slot was freed at the last crossing
#pragma unroll
    for (int u = 1; u < U; ++u) advance(lds + (kt % S) * L::kStage, u);
    cross(kt);
    advance(lds + ((kt + 1) % S) * L::kStage, 0);
  }
#pragma unroll
  for (int u = 1; u < U; ++u) advance(lds + ((nk - 1) % S) * L::kStage, u);
  wait_lds();
  last(bP);
  wait_vm<0>();  // no LDS write may land after the block ends

  // Scales through LDS (free now): as[BM], bs[BN], bb[BN].
  float* sh_as = reinterpret_cast<float*>(lds);
  float* sh_bs = sh_as + BM;
  float* sh_bb = sh_bs + BN;
  block_barrier();  // every wave is done reading the last strip
  if constexpr (OUT != 2) {
    const int t = threadIdx.x;
    if (t < BM) sh_as[t] = pre_as;
    if (t < BN) {
      sh_bs[t] = pre_bs;
      sh_bb[t] = pre_bb;
    }
    __syncthreads();
  }
  float bs[FN], bb[FN];
  if constexpr (OUT != 2) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      bs[j] = sh_bs[col0 + r + 32 * j];
      bb[j] = sh_bb[col0 + r + 32 * j];
    }
  }
  // Element (i, j, v): row m0 + row0 + 32 i + 8 (v / 4) + 4 h + v % 4, column n0 + col0 + 32 j + r.
  auto value = [&](int i, int j, int v, const v4f& as4) {
    return float(acc[i][j][v]) * as4[v % 4] * bs[j] + bb[j];
  };
  auto scales4 = [&](int i, int q) {  // a_scale of rows 32 i + 8 q + 4 h .. +3 of the wave part
    v4f t{};
    if constexpr (OUT != 2) t = *reinterpret_cast<const v4f*>(sh_as + row0 + 32 * i + 8 * q + 4 * h);
    return t;
  };
  if (vec && m0 + BM <= M && n0 + BN <= N) {
    const Slab<OUT, FN, 32> slab{lds + kSlabBase + wid * Slab<OUT, FN, 32>::kBytes, lane};
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f as4 = scales4(i, q);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int row = 8 * q + 4 * h + p, col = 32 * j + r;
            if constexpr (OUT == 2) slab.put_i(row, col, acc[i][j][4 * q + p]);
            else slab.put_f(row, col, value(i, j, 4 * q + p, as4));
          }
      }
      slab.flush(out, N, m0 + row0 + 32 * i, n0 + col0);
      wait_lds();  // slab reads done before it is rewritten
    }
  } else {
    const int64_t mw = m0 + row0 + 4 * h, nw = n0 + col0 + r;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f as4 = scales4(i, q);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int64_t m = mw + 32 * i + 8 * q + p;
          if (m >= M) continue;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int64_t n = nw + 32 * j;
            if (n >= N) continue;
            if constexpr (OUT == 2) reinterpret_cast<int32_t*>(out)[m * N + n] = acc[i][j][4 * q + p];
            else put_out<OUT>(out, m * N + n, value(i, j, 4 * q + p, as4));
          }
        }
      }
  }
}

template <int BM, int BN, int S, int WY, int NW, int SB = 64>
hipError_t launch_fp8_w8a8_cfg2(const uint8_t* a, const uint8_t* b, void* out, int out_bf16, int64_t M, int64_t N,
                                int64_t K, float alpha, hipStream_t s) {
  using L = I8Layout<BM, BN, S, WY, NW, SB>;
  const int64_t blocks = tiles(M, N, BM, BN);
  const int vec = aligned16(out) && (N * (out_bf16 ? 2 : 4)) % 16 == 0;
  if (out_bf16)
    return launch_big_lds<fp8_w8a8_lds2_kernel<BM, BN, S, WY, NW, 1, SB>>(L::kLds, blocks, 64 * NW, s, a, b, out, M, N,
                                                                      K, alpha, vec);
  return launch_big_lds<fp8_w8a8_lds2_kernel<BM, BN, S, WY, NW, 0, SB>>(L::kLds, blocks, 64 * NW, s, a, b, out, M, N, K,
                                                                    alpha, vec);
}

template <int BM, int BN, int S, int WY, int NW>
hipError_t launch_fp8_w8a8_cfg(const uint8_t* a, const uint8_t* b, void* out, int out_bf16, int64_t M, int64_t N,
                               int64_t K, float alpha, hipStream_t s) {
  using L = I8Layout<BM, BN, S, WY, NW>;
  const int64_t blocks = tiles(M, N, BM, BN);
  const int vec = aligned16(out) && (N * (out_bf16 ? 2 : 4)) % 16 == 0;
  if (out_bf16)
    return launch_big_lds<fp8_w8a8_lds_kernel<BM, BN, S, WY, NW, 1>>(L::kLds, blocks, 64 * NW, s, a, b, out, M, N, K,
                                                                     alpha, vec);
  return launch_big_lds<fp8_w8a8_lds_kernel<BM, BN, S, WY, NW, 0>>(L::kLds, blocks, 64 * NW, s, a, b, out, M, N, K,
                                                                   alpha, vec);
}

template <int BM, int BN, int S, int WY, int NW, int SB>
hipError_t launch_int8_lds2(const int8_t* a, const int8_t* b, const float* sa, const float* sb, const uint16_t* bias,
                            void* out, int out_mode, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  using L = I8Layout<BM, BN, S, WY, NW, SB>;
  const int64_t blocks = tiles(M, N, BM, BN);
  const int es = out_mode == 1 ? 2 : 4;
  const int vec = aligned16(out) && (N * es) % 16 == 0;
  switch (out_mode) {
    case 0:
      return launch_big_lds<int8_lds2_kernel<BM, BN, S, WY, NW, 0, SB>>(L::kLds, blocks, 64 * NW, s, a, b, sa, sb, bias,
                                                                        out, M, N, K, vec);
    case 1:
      return launch_big_lds<int8_lds2_kernel<BM, BN, S, WY, NW, 1, SB>>(L::kLds, blocks, 64 * NW, s, a, b, sa, sb, bias,
                                                                        out, M, N, K, vec);
    default:
      return launch_big_lds<int8_lds2_kernel<BM, BN, S, WY, NW, 2, SB>>(L::kLds, blocks, 64 * NW, s, a, b, sa, sb, bias,
                                                                        out, M, N, K, vec);
  }
}

template <int BM, int BN, int S, int WY, int NW, int SB = 64>
hipError_t launch_int8_cfg(const int8_t* a, const int8_t* b, const float* sa, const float* sb, const uint16_t* bias,
                           void* out, int out_mode, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  using L = I8Layout<BM, BN, S, WY, NW, SB>;
  const int64_t blocks = tiles(M, N, BM, BN);
  const int es = out_mode == 1 ? 2 : 4;
  const int vec = aligned16(out) && (N * es) % 16 == 0;
  switch (out_mode) {
    case 0:
      return launch_big_lds<int8_gemm_lds_kernel<BM, BN, S, WY, NW, 0, SB>>(L::kLds, blocks, 64 * NW, s, a, b, sa, sb,
                                                                        bias, out, M, N, K, vec);
    case 1:
      return launch_big_lds<int8_gemm_lds_kernel<BM, BN, S, WY, NW, 1, SB>>(L::kLds, blocks, 64 * NW, s, a, b, sa, sb,
                                                                        bias, out, M, N, K, vec);
    default:
      return launch_big_lds<int8_gemm_lds_kernel<BM, BN, S, WY, NW, 2, SB>>(L::kLds, blocks, 64 * NW, s, a, b, sa, sb,
                                                                        bias, out, M, N, K, vec);
  }
}

}  // namespace

// 32-bit per-lane DMA offsets: every operand must span fewer than 2^32 bytes.
bool gemm_lds_supported(const void* x, const void* w, const void* scales, int64_t M, int64_t N, int64_t K) {
  return K >= 64 && K % 64 == 0 && aligned16(x) && aligned16(w) && reinterpret_cast<uintptr_t>(scales) % 4 == 0 &&
         M * K * 2 < (int64_t(1) << 32) && N * K < (int64_t(1) << 32);
}

bool int8_lds_supported(const void* a, const void* b, int64_t M, int64_t N, int64_t K) {
  return K >= 64 && K % 64 == 0 && aligned16(a) && aligned16(b) && M * K < (int64_t(1) << 32) &&
         N * K < (int64_t(1) << 32);
}

hipError_t launch_fp8_gemm_lds(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                               int64_t K, float alpha, int num_cus, float* ws, size_t ws_bytes, hipStream_t s,
                               const Epilogue& epi) {
  const Fp8Args wa{w};
  if (ws) {
    const int kv = K % 128 == 0 ? 128 : 64;  // values of k per strip
    const int sp = splitk_count(tiles(M, N, 128, 128), M, N, K, kv, num_cus, ws_bytes);
    if (sp > 1) {
      if (kv == 128)
        return launch_wq_splitk<Fp8Weight2, 128, 128, 2, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, sp, ws, epi, s);
      return launch_wq_splitk<Fp8Weight, 128, 128, 4, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, sp, ws, epi, s);
    }
  }
  // Largest tile that still gives every CU a block; 128-value strips (whole
  // weight lines, two stages) where K allows and the LDS holds them
  // (M = 2048, N = K = 4096: 67 against 71-72 us; split-K M = 128: 20.7
  // against 21.1 us).
  if (tiles(M, N, 256, 256) >= num_cus)
    return launch_wq<Fp8Weight, 256, 256, 3, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, epi, s);
  if (tiles(M, N, 256, 128) >= num_cus)
    return K % 128 == 0 ? launch_wq<Fp8Weight2, 256, 128, 2, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, epi, s)
                        : launch_wq<Fp8Weight, 256, 128, 3, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, epi, s);
  return launch_wq<Fp8Weight, 128, 128, 4, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, epi, s);
}

hipError_t launch_nvfp4_gemm_lds(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* out,
                                 int out_bf16, int64_t M, int64_t N, int64_t K, float alpha, int num_cus, float* ws,
                                 size_t ws_bytes, hipStream_t s, const Epilogue& epi) {
  const Nvfp4Args wa{packed, scales};
  if (ws) {
    // Up to 256 rows, 64-row tiles with four waves side by side (no weight
    // row decoded twice) and half the partial planes of 128-row tiles
    // (M = 128, N = K = 4096: 22.2 -> 18.4 us); larger M keeps 128 x 128.
    if (M <= 256) {
      const int kv = K % 128 == 0 ? 128 : 64;
      const int sp = splitk_count(tiles(M, N, 64, 128), M, N, K, kv, num_cus, ws_bytes);
      if (sp > 1 && kv == 128)  // 128-value strips: M = 128 17.7 against 18.5 us
        return launch_wq_splitk<Nvfp4Weight2, 64, 128, 2, 1, 4>(x, wa, out, out_bf16, M, N, K, alpha, sp, ws, epi, s);
      if (sp > 1)
        return launch_wq_splitk<Nvfp4Weight, 64, 128, 4, 1, 4>(x, wa, out, out_bf16, M, N, K, alpha, sp, ws, epi, s);
    }
    const int sp = splitk_count(tiles(M, N, 128, 128), M, N, K, 64, num_cus, ws_bytes);
    if (sp > 1)
      return launch_wq_splitk<Nvfp4Weight, 128, 128, 4, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, sp, ws, epi, s);
  }
  // The FP4 decode is the expensive part: waves side by side along N (WY = 1)
  // where the tile is wide enough, so that no two waves decode the same
  // weight rows.  With a 256 x 256 tile for every CU, its halved L2 -> LDS
  // traffic wins instead (M = N = K = 4096: 156 -> 143 us).
  if (tiles(M, N, 256, 256) >= num_cus)
    return launch_wq<Nvfp4Weight, 256, 256, 3, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, epi, s);
  // Where K allows, 128-value strips (64 packed bytes per weight row) in a
  // two-stage ring: M = 2048, N = K = 4096 70 against 73 us with a few
  // weight copies, the same 75 us with weights cycled through 1 GiB (three
  // stages: 74 us).  Taken while more than half of the CUs get a tile.
  if (tiles(M, N, 128, 256) > num_cus / 2) {
    if (K % 128 == 0) return launch_wq<Nvfp4Weight2, 128, 256, 2, 1, 8>(x, wa, out, out_bf16, M, N, K, alpha, epi, s);
    return launch_wq<Nvfp4Weight, 128, 256, 4, 1, 8>(x, wa, out, out_bf16, M, N, K, alpha, epi, s);
  }
  // Fewer tiles: 128 x 128 with four waves side by side (each 128 x 32, no
  // weight row decoded twice) and 64-value strips in a two-stage ring, 41
  // KiB of LDS, so that two or three blocks share a CU.  M = 1024, N = K =
  // 4096: 49.6 against 61.4 us for 128 x 256 tiles on half of the CUs; at M
  // = 256 .. 768 without split-K within 1 us of 128 x 128 with 2 x 4 waves
  // and four stages, which it replaces.
  return launch_wq<Nvfp4Weight, 128, 128, 2, 1, 4>(x, wa, out, out_bf16, M, N, K, alpha, epi, s);
}

// Workspace bytes with which the launchers above take their split-K kernels
// for (M, N, K) on a device with num_cus CUs (0: they run whole-K tiles).
// These mirror the launchers' own choice made with an unbounded workspace.
// The workspace each launch above asks for (the same slice counts).
size_t fp8_gemm_lds_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus) {
  const int kv = K % 128 == 0 ? 128 : 64;
  return planes_bytes(splitk_count(tiles(M, N, 128, 128), M, N, K, kv, num_cus, SIZE_MAX), M, N);
}

size_t nvfp4_gemm_lds_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus) {
  if (M <= 256) {
    const int sp = splitk_count(tiles(M, N, 64, 128), M, N, K, K % 128 == 0 ? 128 : 64, num_cus, SIZE_MAX);
    if (sp > 1) return planes_bytes(sp, M, N);
  }
  return planes_bytes(splitk_count(tiles(M, N, 128, 128), M, N, K, 64, num_cus, SIZE_MAX), M, N);
}

size_t bf16_gemm_lds_ws_bytes(int64_t M, int64_t N, int64_t K, int num_cus) {
  return planes_bytes(splitk_count(tiles(M, N, 128, 128), M, N, K, 64, num_cus, SIZE_MAX), M, N);
}

hipError_t launch_splitk_reduce(const float* part, void* out, int out_bf16, int64_t M, int64_t N, int splits,
                                float alpha, hipStream_t s, const Epilogue& epi) {
  const int64_t count = M * N, rblocks = (count + 1023) / 1024;
  if (out_bf16)
    return launch(wq_reduce_kernel<1>, dim3(rblocks), dim3(256), 0, s, part, out, count, splits, alpha, N, epi);
  return launch(wq_reduce_kernel<0>, dim3(rblocks), dim3(256), 0, s, part, out, count, splits, alpha, N, epi);
}

bool bf16_lds_supported(const void* x, const void* w, int64_t M, int64_t N, int64_t K) {
  return K >= 64 && K % 64 == 0 && aligned16(x) && aligned16(w) && M * K * 2 < (int64_t(1) << 32) &&
         N * K * 2 < (int64_t(1) << 32);
}

hipError_t launch_bf16_gemm_lds(const uint16_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                                int64_t K, float alpha, int num_cus, float* ws, size_t ws_bytes, hipStream_t s,
                                const Epilogue& epi) {
  const Bf16Args wa{w};
  if (ws) {
    const int sp = splitk_count(tiles(M, N, 128, 128), M, N, K, 64, num_cus, ws_bytes);
    if (sp > 1) return launch_wq_splitk<Bf16Weight, 128, 128, 4, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, sp, ws, epi, s);
  }
  // A 256 x 256 stage of both bf16 operands (64 KiB) leaves room for only two
  // stages: the largest tile runs 256 x 128 with three.
  if (tiles(M, N, 256, 128) >= num_cus)
    return launch_wq<Bf16Weight, 256, 128, 3, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, epi, s);
  return launch_wq<Bf16Weight, 128, 128, 4, 2, 8>(x, wa, out, out_bf16, M, N, K, alpha, epi, s);
}

namespace {

// Grouped tile: BM x BN with NW waves.  Short groups waste little of a
// tall tile: their missing rows are zero-filled without traffic and waves
// past a group's last row only fetch.
template <template <int, int, int> class WP, int BM, int BN, int S, int WY, int NW>
hipError_t launch_grouped_cfg(typename WP<BN, 1, NW>::Args wa, const uint16_t* x, const uint32_t* a_offsets,
                              const int32_t* expert_ids, void* out, int out_bf16, int64_t G, int64_t E, int64_t T,
                              int64_t N, int64_t K, int num_cus, hipStream_t s, const float* expert_scale) {
  using L = WqLayout<WP, BM, BN, S, WY, NW>;
  const int lds_bytes = int(L::kLds + 4 * (G + 1));
  if (lds_bytes > kMaxLds) return hipErrorInvalidValue;
  // At most ceil(T / BM) + G row tiles exist; as many blocks as fit on the
  // CUs walk them.  The kernel splits the work over 8 XCDs: a multiple of 8.
  const int64_t upper = ((T + BM - 1) / BM + G) * ((N + BN - 1) / BN);
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(kMaxLds / lds_bytes, 16 / NW));
  const int64_t want = upper < per_cu * num_cus ? upper : per_cu * num_cus;
  const int64_t blocks = (want + 7) / 8 * 8;
  const int es = out_bf16 ? 2 : 4;
  const int vec = aligned16(out) && (N * es) % 16 == 0;
  auto go = [&](auto kernel) -> hipError_t {
    // The LDS size depends on G: raise the kernel's limit to the maximum once.
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kernel), kMaxLds, lds_set)) return e;
    return launch(kernel, dim3(blocks), dim3(64 * NW), lds_bytes, s, x, wa, a_offsets, expert_ids, expert_scale, out, G,
                  T, N, K, E, vec);
  };
  if (out_bf16) return go(grouped_gemm_kernel<WP, BM, BN, S, WY, NW, 1>);
  return go(grouped_gemm_kernel<WP, BM, BN, S, WY, NW, 0>);
}

constexpr int kGrpBM = 64, kGrpBN = 128, kGrpS = 4, kGrpWY = 2, kGrpNW = 4;
using GrpLayout = WqLayout<Fp8Weight, kGrpBM, kGrpBN, kGrpS, kGrpWY, kGrpNW>;
// NVFP4 experts: 64 x 256 tiles, eight waves side by side along N (each
// 64 x 32), so no two waves decode the same weight rows (measured 5-10 %
// faster than 2 x 2) and each activation strip feeds 256 columns (about 6 %
// faster than 64 x 128 on the 64-expert workload).
constexpr int kGrp4BN = 256, kGrp4WY = 1, kGrp4NW = 8;
using GrpLayoutFp4 = WqLayout<Nvfp4Weight, kGrpBM, kGrp4BN, kGrpS, kGrp4WY, kGrp4NW>;

}  // namespace

bool grouped_lds_supported(const void* x, const void* w, int64_t G, int64_t T, int64_t N, int64_t K) {
  return K >= 64 && K % 64 == 0 && aligned16(x) && aligned16(w) && T * K * 2 < (int64_t(1) << 32) &&
         N * K < (int64_t(1) << 32) && GrpLayout::kLds + 4 * (G + 1) <= kMaxLds &&
         (T + G) * ((N + kGrpBN - 1) / kGrpBN) < (int64_t(1) << 31);
}

bool nvfp4_grouped_lds_supported(const void* x, const void* packed, const void* scales, int64_t G, int64_t T,
                                 int64_t N, int64_t K) {
  return K >= 64 && K % 64 == 0 && aligned16(x) && aligned16(packed) &&
         reinterpret_cast<uintptr_t>(scales) % 4 == 0 && T * K * 2 < (int64_t(1) << 32) &&
         N * (K / 2) < (int64_t(1) << 32) && GrpLayoutFp4::kLds + 4 * (G + 1) <= kMaxLds &&
         (T + G) * ((N + kGrp4BN - 1) / kGrp4BN) < (int64_t(1) << 31);
}

hipError_t launch_fp8_grouped_lds(const uint8_t* w, const uint16_t* x, const uint32_t* a_offsets,
                                  const int32_t* expert_ids, void* out, int out_bf16, int64_t G, int64_t E, int64_t T,
                                  int64_t N, int64_t K, int num_cus, hipStream_t s, const float* expert_scale) {
  // Where K allows, 128-value strips (whole 128-byte weight lines) in a
  // two-stage ring, the same 64 KiB of LDS: 64 against 68 us on the
  // 64-expert workload (a three-stage ring, one block per CU: 82 us).
  if (K % 128 == 0)
    return launch_grouped_cfg<Fp8Weight2, kGrpBM, kGrpBN, 2, kGrpWY, kGrpNW>(
        Fp8Args{w}, x, a_offsets, expert_ids, out, out_bf16, G, E, T, N, K, num_cus, s, expert_scale);
  return launch_grouped_cfg<Fp8Weight, kGrpBM, kGrpBN, kGrpS, kGrpWY, kGrpNW>(
      Fp8Args{w}, x, a_offsets, expert_ids, out, out_bf16, G, E, T, N, K, num_cus, s, expert_scale);
}

hipError_t launch_nvfp4_grouped_lds(const uint8_t* packed, const uint8_t* scales, const uint16_t* x,
                                    const uint32_t* a_offsets, const int32_t* expert_ids, void* out, int out_bf16,
                                    int64_t G, int64_t E, int64_t T, int64_t N, int64_t K, int num_cus,
                                    hipStream_t s, const float* expert_scale) {
  // 128-value strips in a two-stage ring where K allows: 65 against 76 us on
  // the 64-expert workload.
  if (K % 128 == 0)
    return launch_grouped_cfg<Nvfp4Weight2, kGrpBM, kGrp4BN, 2, kGrp4WY, kGrp4NW>(
        Nvfp4Args{packed, scales}, x, a_offsets, expert_ids, out, out_bf16, G, E, T, N, K, num_cus, s, expert_scale);
  return launch_grouped_cfg<Nvfp4Weight, kGrpBM, kGrp4BN, kGrpS, kGrp4WY, kGrp4NW>(
      Nvfp4Args{packed, scales}, x, a_offsets, expert_ids, out, out_bf16, G, E, T, N, K, num_cus, s, expert_scale);
}

hipError_t launch_fp8_w8a8_lds(const uint8_t* xq, const uint8_t* w, void* out, int out_bf16, int64_t M, int64_t N,
                               int64_t K, float alpha, int num_cus, hipStream_t s) {
  // The 256 x 256 tile needs the in-place fragment refresh of
  // fp8_w8a8_lds2_kernel to fit two waves per SIMD (4096 x 12288 x 3072:
  // 175 us against 199 us for 256 x 128).
  if (tiles(M, N, 256, 256) >= num_cus / 2) {
    if (K % 128 == 0) return launch_fp8_w8a8_cfg2<256, 256, 2, 2, 8, 128>(xq, w, out, out_bf16, M, N, K, alpha, s);
    return launch_fp8_w8a8_cfg2<256, 256, 4, 2, 8>(xq, w, out, out_bf16, M, N, K, alpha, s);
  }
  if (tiles(M, N, 256, 128) >= num_cus / 2)
    return launch_fp8_w8a8_cfg<256, 128, 4, 2, 8>(xq, w, out, out_bf16, M, N, K, alpha, s);
  return launch_fp8_w8a8_cfg<128, 128, 4, 2, 8>(xq, w, out, out_bf16, M, N, K, alpha, s);
}

hipError_t launch_int8_gemm_lds(const int8_t* a, const int8_t* b, const float* sa, const float* sb,
                                const uint16_t* bias, void* out, int out_mode, int64_t M, int64_t N, int64_t K,
                                int num_cus, hipStream_t s) {
  // 256 x 256 tiles halve the L2 -> LDS traffic of 256 x 128 ones, which
  // pays even when some CUs get no tile.  128-byte strips (two stages in the
  // ring) beat 64-byte ones (four stages) where K allows: 4096 x 12288 x
  // 3072 147 against 158 us, 4096 x 3072 x 3072 42.5 against 45.8 us.  With
  // such strips the W8A8 structure (split DMA, fragments refreshed in place)
  // is about 1 % faster again: 138.9 against 140.1 us, 40.9 against 41.2 us.
  if (tiles(M, N, 256, 256) >= num_cus / 2) {
    if (K % 128 == 0)
      return launch_int8_lds2<256, 256, 2, 2, 8, 128>(a, b, sa, sb, bias, out, out_mode, M, N, K, s);
    return launch_int8_cfg<256, 256, 4, 2, 8>(a, b, sa, sb, bias, out, out_mode, M, N, K, s);
  }
  if (tiles(M, N, 256, 128) >= num_cus / 2)
    return launch_int8_cfg<256, 128, 4, 2, 8>(a, b, sa, sb, bias, out, out_mode, M, N, K, s);
  return launch_int8_cfg<128, 128, 4, 2, 8>(a, b, sa, sb, bias, out, out_mode, M, N, K, s);
}

namespace {

template <int BM, int BN, int S, int WY, int NW, int SB = 64>
hipError_t launch_int8_grouped_cfg(const int8_t* a, const int8_t* b, const float* sa, const float* sb,
                                   const uint16_t* bias, const uint32_t* a_offsets, const int32_t* expert_ids,
                                   void* out, int out_mode, int64_t G, int64_t E, int64_t T, int64_t N, int64_t K,
                                   int num_cus, hipStream_t s) {
  using L = I8Layout<BM, BN, S, WY, NW, SB>;
  const int lds_bytes = int(L::kLds + 4 * (G + 1));
  if (lds_bytes > kMaxLds) return hipErrorInvalidValue;
  const int64_t upper = ((T + BM - 1) / BM + G) * ((N + BN - 1) / BN);
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(kMaxLds / lds_bytes, 16 / NW));
  const int64_t want = upper < per_cu * num_cus ? upper : per_cu * num_cus;
  const int64_t blocks = (want + 7) / 8 * 8;
  const int es = out_mode == 1 ? 2 : 4;
  const int vec = aligned16(out) && (N * es) % 16 == 0;
  auto go = [&](auto kernel) -> hipError_t {
    static std::atomic<uint64_t> lds_set{0};
    if (hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kernel), kMaxLds, lds_set)) return e;
    return launch(kernel, dim3(blocks), dim3(64 * NW), lds_bytes, s, a, b, sa, sb, bias, a_offsets, expert_ids, out,
                  G, T, N, K, E, vec);
  };
  if (out_mode == 1) return go(int8_grouped_kernel<BM, BN, S, WY, NW, 1, SB>);
  if (out_mode == 2) return go(int8_grouped_kernel<BM, BN, S, WY, NW, 2, SB>);
  return go(int8_grouped_kernel<BM, BN, S, WY, NW, 0, SB>);
}

}  // namespace

bool int8_grouped_lds_supported(const void* a, const void* b, int64_t G, int64_t T, int64_t N, int64_t K) {
  return K >= 64 && K % 64 == 0 && aligned16(a) && aligned16(b) && T * K < (int64_t(1) << 32) &&
         N * K < (int64_t(1) << 32) && G <= 8192;
}

hipError_t launch_int8_grouped_lds(const int8_t* a, const int8_t* b, const float* sa, const float* sb,
                                   const uint16_t* bias, const uint32_t* a_offsets, const int32_t* expert_ids,
                                   void* out, int out_mode, int64_t G, int64_t E, int64_t T, int64_t N, int64_t K,
                                   int num_cus, hipStream_t s) {
  // The grouped W8A16 tile shape: 64 rows (groups average ~64 tokens), 128
  // columns, four waves side by side.  Where K allows, 128-byte strips in a
  // two-stage ring (the same 48 KiB of LDS, three blocks per CU): 49 against
  // 62 us on the 64-expert workload (a three-stage ring: 52 us).
  if (K % 128 == 0)
    return launch_int8_grouped_cfg<64, 128, 2, 1, 4, 128>(a, b, sa, sb, bias, a_offsets, expert_ids, out, out_mode, G,
                                                          E, T, N, K, num_cus, s);
  return launch_int8_grouped_cfg<64, 128, 4, 1, 4>(a, b, sa, sb, bias, a_offsets, expert_ids, out, out_mode, G, E, T,
                                                   N, K, num_cus, s);
}

}  // namespace qlinear
