// Pipelined LDS GEMMs for large problems:
//   * W8A16 / W4A16:  out[m, n] = alpha * sum_k x[m, k] * dec(W[n, k]),  K % 64 == 0
//     ("Matmul2dFp8" page, W8A16 GEMM; "fp4_matmul" page, W4A16 GEMM with the
//     weight sub-tile dequantised to bfloat16 once per K strip, cooperatively
//     by the whole block, into on-chip memory)
//   * W8A8 int8:      acc = a @ b^T (int32), out = acc * a_scale[m] * b_scale[n] + bias[n],
//     K % 128 == 0 ("int8_matmul" page)
// These are the fast paths for aligned operands; gemm_bf16.hip / int8.hip
// serve every other shape.
//
// gfx950 structure:
// * A 256-thread block (2 x 2 waves) owns a BM x BN output tile and walks K
//   in strips of 128 bytes per activation row (64 bf16 or 128 int8 values)
//   through an S-stage ring of LDS buffers.
// * Strips are fetched with global_load_lds_dwordx4: the load unit writes
//   each lane's 16 bytes straight into LDS (lane i at base + 16 i), so no
//   registers stage the data and S - 1 strips are in flight while the
//   matrix cores work on the current one.  Which global chunk each lane
//   fetches is chosen so that the 16-byte chunks of a row land XOR-swizzled
//   by row index (slot = chunk ^ (row % 8)), which keeps the 16-row fragment
//   reads free of LDS bank conflicts.  Each lane's address is a uniform
//   strip base plus a 32-bit offset computed once per block.
// * The quantized weight strip lands in its stored form (fp8 bytes, or packed
//   fp4 + E4M3 scales); all 256 threads then decode it once into a bfloat16
//   tile in the same swizzled layout (exact decode, FP4 block scale applied in
//   float32), and the waves read both operands with 16-byte LDS reads for
//   v_mfma_f32_16x16x32_bf16.  int8 strips need no decode and feed
//   v_mfma_i32_16x16x64_i8 directly.
// * Rows past M or N are fetched from the last valid row (the DMA cannot
//   zero-fill); they only feed outputs that are not stored.
#include "device.hpp"
#include "launch.hpp"

namespace qlinear {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int kThreads = 256;
constexpr int kRow = 128;  // bytes per row of every LDS operand tile (8 chunks of 16 B)

__device__ __forceinline__ void dma16(const char* g, char* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const char* g, char* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds, 4, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// the fences would wait for every outstanding vector-memory operation,
// including the strips still in flight.  The DMA writes of the strip being
// consumed are complete (wait_vm before the barrier) and the asm statements
// keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- 128-byte-row strips

// Per-lane DMA offsets for a strip of 128 bytes per row of a row-major
// operand (row stride `row_bytes`), rows r0 .. r0 + ROWS - 1 clipped to `rows`:
// instruction q of wave w covers rows 8 (4q + w) .. +7; lane i -> row +i/8,
// LDS slot i%8 holding global chunk slot ^ (row % 8).
template <int ROWS>
struct Rows128 {
  static constexpr int kInst = ROWS / 32;  // DMA instructions per wave per strip
  uint32_t off[kInst];
  __device__ __forceinline__ void init(int64_t r0, int64_t rows, int64_t row_bytes) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int r = 8 * (4 * q + wid) + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);
      int64_t row = r0 + r;
      if (row >= rows) row = rows - 1;
      off[q] = uint32_t(row * row_bytes + 16 * c);
    }
  }
  // base = operand start + the strip's byte offset within a row (uniform)
  __device__ __forceinline__ void fetch(char* lds, const char* base) const {
    const int wid = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kInst; ++q) dma16(base + off[q], lds + 8 * (4 * q + wid) * kRow);
  }
};

// Fragment read of a 128-byte-row tile: lane (r16, g) of 16-row group i,
// k-step ks reads chunk 4 ks + g of row row0 + 16 i + r16.  (row0 is a
// multiple of 8, so the swizzle only depends on r16.)
struct FragAddr {
  uint32_t base[2];
  __device__ __forceinline__ void init(int row0, int r16, int g) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) base[ks] = uint32_t((row0 + r16) * kRow + 16 * ((4 * ks + g) ^ (r16 & 7)));
  }
  __device__ __forceinline__ u32x4 read(const char* tile, int ks, int i) const {
    return *reinterpret_cast<const u32x4*>(tile + base[ks] + 16 * kRow * i);
  }
};

// ---------------------------------------------------------------- weight strips (bf16 GEMM)

// fp8 strip: 64 bytes per row.  Instruction q of wave w covers rows
// 16 (4q + w) .. +15: lane i -> row +i/4, raw chunk i%4 (unswizzled: the raw
// strip is only read by the decode pass).
template <int BN>
struct Fp8Strip {
  static constexpr int kBytes = BN * 64;
  static constexpr int kInst = BN / 64;
  uint32_t off[kInst];
  __device__ __forceinline__ void init(int64_t n0, int64_t N, int64_t K) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int r = 16 * (4 * q + wid) + (lane >> 2);
      int64_t n = n0 + r;
      if (n >= N) n = N - 1;
      off[q] = uint32_t(n * K + 16 * (lane & 3));
    }
  }
  __device__ __forceinline__ void fetch(char* lds, const uint8_t* w, const uint8_t*, int64_t k0) const {
    const int wid = threadIdx.x >> 6;
    const char* base = reinterpret_cast<const char*>(w) + k0;
#pragma unroll
    for (int q = 0; q < kInst; ++q) dma16(base + off[q], lds + 16 * (4 * q + wid) * 64);
  }
  // Decode the raw strip into the swizzled bf16 tile, one raw 16-byte chunk
  // (two bf16 chunks) per thread per step.
  __device__ __forceinline__ void decode(char* dst, const char* raw) const {
#pragma unroll
    for (int p = 0; p < BN * 4 / kThreads; ++p) {
      const int id = threadIdx.x + kThreads * p;  // raw chunk id
      const int r = id >> 2, c = id & 3;          // row, raw chunk (k = 16 c .. +15)
      const u32x4 v = *reinterpret_cast<const u32x4*>(raw + r * 64 + 16 * c);
      const u32x4 lo{e4m3x2_to_bf16x2<false>(v.x), e4m3x2_to_bf16x2<true>(v.x),
                     e4m3x2_to_bf16x2<false>(v.y), e4m3x2_to_bf16x2<true>(v.y)};
      const u32x4 hi{e4m3x2_to_bf16x2<false>(v.z), e4m3x2_to_bf16x2<true>(v.z),
                     e4m3x2_to_bf16x2<false>(v.w), e4m3x2_to_bf16x2<true>(v.w)};
      *reinterpret_cast<u32x4*>(dst + r * kRow + 16 * ((2 * c) ^ (r & 7))) = lo;
      *reinterpret_cast<u32x4*>(dst + r * kRow + 16 * ((2 * c + 1) ^ (r & 7))) = hi;
    }
  }
};

// NVFP4 strip: 32 packed bytes + 4 scale bytes per row.  Packed: instruction
// q of wave w covers rows 32 (4q + w) .. +31, lane i -> row +i/2, raw chunk
// i%2.  Scales: 32 rows per instruction with lanes 0..31 (one dword each).
template <int BN>
struct Nvfp4Strip {
  static constexpr int kPacked = BN * 32;
  static constexpr int kBytes = BN * 36;
  static constexpr int kInst = 2 * (BN / 128);  // packed + scale instructions per wave
  uint32_t poff[BN / 128], soff[BN / 128];
  __device__ __forceinline__ void init(int64_t n0, int64_t N, int64_t K) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < BN / 128; ++q) {
      const int r = 32 * (4 * q + wid) + (lane >> 1);
      int64_t n = n0 + r;
      if (n >= N) n = N - 1;
      poff[q] = uint32_t(n * (K >> 1) + 16 * (lane & 1));
      int64_t ns = n0 + 32 * (4 * q + wid) + (lane & 31);
      if (ns >= N) ns = N - 1;
      soff[q] = uint32_t(ns * (K >> 4));
    }
  }
  __device__ __forceinline__ void fetch(char* lds, const uint8_t* packed, const uint8_t* scales, int64_t k0) const {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const char* pb = reinterpret_cast<const char*>(packed) + (k0 >> 1);
    const char* sb = reinterpret_cast<const char*>(scales) + (k0 >> 4);
#pragma unroll
    for (int q = 0; q < BN / 128; ++q) {
      dma16(pb + poff[q], lds + 32 * (4 * q + wid) * 32);
      if (lane < 32) dma4(sb + soff[q], lds + kPacked + 32 * (4 * q + wid) * 4);
    }
  }
  // Thread t decodes 16 packed bytes (32 weights, two scale blocks) into
  // four bf16 chunks of the swizzled tile.
  __device__ __forceinline__ void decode(char* dst, const char* raw) const {
#pragma unroll
    for (int p = 0; p < BN * 2 / kThreads; ++p) {
      const int id = threadIdx.x + kThreads * p;
      const int r = id >> 1, h = id & 1;  // row, half of the 64-wide strip
      const u32x4 v = *reinterpret_cast<const u32x4*>(raw + r * 32 + 16 * h);
      const uint32_t sc = *reinterpret_cast<const uint16_t*>(raw + kPacked + r * 4 + 2 * h);
#pragma unroll
      for (int d = 0; d < 4; ++d) {  // dword d = weights 8 d .. 8 d + 7 of the half
        const float s = e4m3_to_f32((sc >> (8 * (d >> 1))) & 0xFFu);
        const u32x4 o{e2m1x2_to_bf16x2<0>(v[d], s), e2m1x2_to_bf16x2<1>(v[d], s),
                      e2m1x2_to_bf16x2<2>(v[d], s), e2m1x2_to_bf16x2<3>(v[d], s)};
        *reinterpret_cast<u32x4*>(dst + r * kRow + 16 * ((4 * h + d) ^ (r & 7))) = o;
      }
    }
  }
};

struct Fp8Args { const uint8_t* w; };
struct Nvfp4Args { const uint8_t* packed; const uint8_t* scales; };

template <class WA, int BN> struct StripOf;
template <int BN> struct StripOf<Fp8Args, BN> { using type = Fp8Strip<BN>; };
template <int BN> struct StripOf<Nvfp4Args, BN> { using type = Nvfp4Strip<BN>; };
__device__ __forceinline__ const uint8_t* wptr(Fp8Args a) { return a.w; }
__device__ __forceinline__ const uint8_t* wptr(Nvfp4Args a) { return a.packed; }
__device__ __forceinline__ const uint8_t* sptr(Fp8Args) { return nullptr; }
__device__ __forceinline__ const uint8_t* sptr(Nvfp4Args a) { return a.scales; }

// Block b -> (row tile, column tile).  Blocks are dealt to the 8 XCDs round
// robin, so XCD x runs blocks x, x + 8, ...; give it a contiguous range of
// tiles, and inside the range walk 8 row tiles per column tile.
__device__ __forceinline__ void tile_of_block(int64_t b, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
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

// ---------------------------------------------------------------- bf16 GEMM with decoded weight

template <int BM, int BN, int S, class WS>
struct Layout {
  static constexpr int kA = BM * kRow;
  static constexpr int kStage = kA + WS::kBytes;
  static constexpr int kDec = S * kStage;  // decoded bf16 weight tile after the ring
  static constexpr int kLds = kDec + BN * kRow;
  static constexpr int kLoads = Rows128<BM>::kInst + WS::kInst;
};

template <class WA, int BM, int BN, int S>
__global__ __launch_bounds__(kThreads) void gemm_lds_kernel(const uint16_t* __restrict__ x, WA wa,
                                                            void* __restrict__ out, int out_bf16, int64_t M,
                                                            int64_t N, int64_t K, float alpha) {
  using WS = typename StripOf<WA, BN>::type;
  using L = Layout<BM, BN, S, WS>;
  constexpr int TM = BM / 32, TN = BN / 32;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int64_t tm, tn;
  tile_of_block(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wy = wid >> 1, wx = wid & 1;
  const int r16 = lane & 15, g = lane >> 4;

  Rows128<BM> afetch;
  afetch.init(m0, M, 2 * K);
  WS wfetch;
  wfetch.init(n0, N, K);
  FragAddr fa, fb;
  fa.init(wy * (BM / 2), r16, g);
  fb.init(wx * (BN / 2), r16, g);
  const char* xb = reinterpret_cast<const char*>(x);
  const uint8_t* wp = wptr(wa);
  const uint8_t* sp = sptr(wa);
  char* dec = lds + L::kDec;

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t nk = K / 64;
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    if (s < nk) {
      char* st = lds + s * L::kStage;
      afetch.fetch(st, xb + int64_t(s) * 128);
      wfetch.fetch(st + L::kA, wp, sp, int64_t(s) * 64);
    }
  }
  for (int64_t kt = 0; kt < nk; ++kt) {
    if (nk - 1 - kt >= S - 2) wait_vm<(S - 2) * L::kLoads>();
    else wait_vm<0>();
    block_barrier();  // strip kt has landed for every wave; the decoded tile of strip kt-1 is no longer read
    if (kt + S - 1 < nk) {
      char* st = lds + ((kt + S - 1) % S) * L::kStage;
      afetch.fetch(st, xb + (kt + S - 1) * 128);
      wfetch.fetch(st + L::kA, wp, sp, (kt + S - 1) * 64);
    }
    const char* sa = lds + (kt % S) * L::kStage;
    wfetch.decode(dec, sa + L::kA);
    block_barrier();  // decoded weight tile complete
    u32x4 a[2][TM], b[2][TN];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < TM; ++i) a[ks][i] = fa.read(sa, ks, i);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[ks][j] = fb.read(dec, ks, j);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[ks][i]),
                                                              __builtin_bit_cast(v8bf, b[ks][j]), acc[i][j], 0, 0,
                                                              0);
  }

  // acc[i][j][v] = C[m0 + (BM/2) wy + 16 i + 4 g + v][n0 + (BN/2) wx + 16 j + r16]
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + wy * (BM / 2) + 16 * i + 4 * g + v;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wx * (BN / 2) + 16 * j + r16;
        if (n < N) store_out(out, m * N + n, acc[i][j][v], alpha, out_bf16);
      }
    }
}

template <class WA, int BM, int BN, int S>
hipError_t launch_cfg(const uint16_t* x, WA wa, void* out, int out_bf16, int64_t M, int64_t N, int64_t K,
                      float alpha, hipStream_t s) {
  using L = Layout<BM, BN, S, typename StripOf<WA, BN>::type>;
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_lds_kernel<WA, BM, BN, S>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, L::kLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return launch(gemm_lds_kernel<WA, BM, BN, S>, dim3(blocks), dim3(kThreads), L::kLds, s, x, wa, out, out_bf16, M,
                N, K, alpha);
}

template <class WA>
hipError_t launch_shape(const uint16_t* x, WA wa, void* out, int out_bf16, int64_t M, int64_t N, int64_t K,
                        float alpha, int num_cus, hipStream_t s) {
  // Largest tile that still gives every CU a block.
  const int64_t t256 = ((M + 255) / 256) * ((N + 127) / 128);
  if (t256 >= num_cus) return launch_cfg<WA, 256, 128, 3>(x, wa, out, out_bf16, M, N, K, alpha, s);
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (t128 >= num_cus) return launch_cfg<WA, 128, 128, 4>(x, wa, out, out_bf16, M, N, K, alpha, s);
  return launch_cfg<WA, 64, 128, 4>(x, wa, out, out_bf16, M, N, K, alpha, s);
}

// ---------------------------------------------------------------- W8A8 int8

// out_mode 0 = fp32, 1 = bf16 (dequantised), 2 = raw int32 accumulators.
template <int BM, int BN, int S>
__global__ __launch_bounds__(kThreads) void int8_gemm_lds_kernel(const int8_t* __restrict__ a,
                                                                 const int8_t* __restrict__ b,
                                                                 const float* __restrict__ a_scale,
                                                                 const float* __restrict__ b_scale,
                                                                 const uint16_t* __restrict__ bias,
                                                                 void* __restrict__ out, int out_mode, int64_t M,
                                                                 int64_t N, int64_t K) {
  constexpr int kA = BM * kRow, kB = BN * kRow, kStage = kA + kB;
  constexpr int kLoads = Rows128<BM>::kInst + Rows128<BN>::kInst;
  constexpr int TM = BM / 32, TN = BN / 32;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int64_t tm, tn;
  tile_of_block(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wy = wid >> 1, wx = wid & 1;
  const int r16 = lane & 15, g = lane >> 4;

  Rows128<BM> afetch;
  afetch.init(m0, M, K);
  Rows128<BN> bfetch;
  bfetch.init(n0, N, K);
  FragAddr fa, fb;
  fa.init(wy * (BM / 2), r16, g);
  fb.init(wx * (BN / 2), r16, g);
  const char* pa = reinterpret_cast<const char*>(a);
  const char* pb = reinterpret_cast<const char*>(b);

  v4i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int64_t nk = K / 128;
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    if (s < nk) {
      char* st = lds + s * kStage;
      afetch.fetch(st, pa + int64_t(s) * 128);
      bfetch.fetch(st + kA, pb + int64_t(s) * 128);
    }
  }
  for (int64_t kt = 0; kt < nk; ++kt) {
    if (nk - 1 - kt >= S - 2) wait_vm<(S - 2) * kLoads>();
    else wait_vm<0>();
    block_barrier();
    if (kt + S - 1 < nk) {
      char* st = lds + ((kt + S - 1) % S) * kStage;
      afetch.fetch(st, pa + (kt + S - 1) * 128);
      bfetch.fetch(st + kA, pb + (kt + S - 1) * 128);
    }
    const char* sa = lds + (kt % S) * kStage;
    const char* sb = sa + kA;
    u32x4 xa[2][TM], xb[2][TN];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < TM; ++i) xa[ks][i] = fa.read(sa, ks, i);
#pragma unroll
      for (int j = 0; j < TN; ++j) xb[ks][j] = fb.read(sb, ks, j);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, xa[ks][i]),
                                                            __builtin_bit_cast(v4i, xb[ks][j]), acc[i][j], 0, 0, 0);
  }

  float bs[TN], bb[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t n = n0 + wx * (BN / 2) + 16 * j + r16;
    bs[j] = (out_mode != 2 && n < N) ? b_scale[n] : 0.f;
    bb[j] = (out_mode != 2 && bias && n < N) ? bf16_to_f32(bias[n]) : 0.f;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + wy * (BM / 2) + 16 * i + 4 * g + v;
      if (m >= M) continue;
      const float as = out_mode != 2 ? a_scale[m] : 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wx * (BN / 2) + 16 * j + r16;
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

template <int BM, int BN, int S>
hipError_t launch_int8_cfg(const int8_t* a, const int8_t* b, const float* sa, const float* sb, const uint16_t* bias,
                           void* out, int out_mode, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  constexpr int kLds = S * (BM + BN) * kRow;
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&int8_gemm_lds_kernel<BM, BN, S>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  return launch(int8_gemm_lds_kernel<BM, BN, S>, dim3(blocks), dim3(kThreads), kLds, s, a, b, sa, sb, bias, out,
                out_mode, M, N, K);
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

// 32-bit per-lane DMA offsets: every operand must span fewer than 2^32 bytes.
bool gemm_lds_supported(const void* x, const void* w, const void* scales, int64_t M, int64_t N, int64_t K) {
  return K % 64 == 0 && aligned16(x) && aligned16(w) && reinterpret_cast<uintptr_t>(scales) % 4 == 0 &&
         M * K * 2 < (int64_t(1) << 32) && N * K < (int64_t(1) << 32);
}

bool int8_lds_supported(const void* a, const void* b, int64_t M, int64_t N, int64_t K) {
  return K % 128 == 0 && aligned16(a) && aligned16(b) && M * K < (int64_t(1) << 32) && N * K < (int64_t(1) << 32);
}

hipError_t launch_fp8_gemm_lds(const uint8_t* w, const uint16_t* x, void* out, int out_bf16, int64_t M, int64_t N,
                               int64_t K, float alpha, int num_cus, hipStream_t s) {
  return launch_shape(x, Fp8Args{w}, out, out_bf16, M, N, K, alpha, num_cus, s);
}

hipError_t launch_nvfp4_gemm_lds(const uint8_t* packed, const uint8_t* scales, const uint16_t* x, void* out,
                                 int out_bf16, int64_t M, int64_t N, int64_t K, float alpha, int num_cus,
                                 hipStream_t s) {
  return launch_shape(x, Nvfp4Args{packed, scales}, out, out_bf16, M, N, K, alpha, num_cus, s);
}

hipError_t launch_int8_gemm_lds(const int8_t* a, const int8_t* b, const float* sa, const float* sb,
                                const uint16_t* bias, void* out, int out_mode, int64_t M, int64_t N, int64_t K,
                                int num_cus, hipStream_t s) {
  const int64_t t256 = ((M + 255) / 256) * ((N + 127) / 128);
  if (t256 >= 4 * int64_t(num_cus))
    return launch_int8_cfg<256, 128, 3>(a, b, sa, sb, bias, out, out_mode, M, N, K, s);
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (t128 >= num_cus) return launch_int8_cfg<128, 128, 4>(a, b, sa, sb, bias, out, out_mode, M, N, K, s);
  return launch_int8_cfg<64, 128, 4>(a, b, sa, sb, bias, out, out_mode, M, N, K, s);
}

}  // namespace qlinear
