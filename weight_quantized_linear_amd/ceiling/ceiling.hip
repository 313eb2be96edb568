// Attainable ceilings of one MI355X, measured by bench.py next to the
// library's kernels: how fast a plain read-only stream can pull a weight of
// a given size out of HBM, and how fast back-to-back matrix-core
// instructions run per data type.  The fp8_gemv page argues that the decode
// GEMV is bound by reading the weight ("WHY it wins at decode"); these
// kernels say what "bound" means on this chip.  Not part of libqlinear's
// ABI; declared in include/qlinear_ceiling.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

// Every 16-byte chunk of buf[0, chunks) is loaded once, non-temporally, the
// way the GEMV loads its weight: a wave takes a span of U KiB that is
// contiguous in memory (U load instructions per lane, each covering 1 KiB,
// all issued before any is used), and the waves of the grid stride over the
// spans.  The XOR of everything read is stored only if it equals `key`,
// which keeps the loads alive without writing anything in practice.
template <int U>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ buf, int64_t chunks,
                                                               uint32_t key, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = int64_t(gridDim.x) * (kThreads / 64);
  const int64_t spans = (chunks + 64 * U - 1) / (64 * U);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t sp = int64_t(blockIdx.x) * (kThreads / 64) + threadIdx.x / 64; sp < spans; sp += waves) {
    const int64_t c0 = sp * 64 * U + lane;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = c0 + 64 * u < chunks ? __builtin_nontemporal_load(buf + c0 + 64 * u) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == key) sink[0] = r;
}

// The same stream through the DMA unit straight into LDS (global_load_lds,
// 16 bytes per lane, non-temporal), as the LDS-staged kernels fetch: each
// wave owns U KiB of LDS, keeps one span of U KiB in flight, and waits for
// it before issuing the next into the same place.
template <int U>
__global__ __launch_bounds__(kThreads) void stream_dma_kernel(const char* __restrict__ buf, int64_t chunks,
                                                              uint32_t key, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) char ring[kThreads / 64][U * 1024];
  const int lane = threadIdx.x & 63, wid = threadIdx.x / 64;
  const int64_t waves = int64_t(gridDim.x) * (kThreads / 64);
  const int64_t spans = (chunks + 64 * U - 1) / (64 * U);
  for (int64_t sp = int64_t(blockIdx.x) * (kThreads / 64) + wid; sp < spans; sp += waves) {
    const int64_t c0 = sp * 64 * U + lane;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + 64 * u < chunks ? c0 + 64 * u : chunks - 1;
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) const void*)(buf + 16 * c),
                                       (__attribute__((address_space(3))) void*)(&ring[wid][u * 1024]), 16, 0, 2);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const uint32_t r = *reinterpret_cast<const uint32_t*>(&ring[wid][16 * lane]);
  if (r == key) sink[0] = r;
}

// L2 -> CU rate: every wave re-reads `iters` spans of U KiB of a small
// buffer (resident in each XCD's L2 after the first pass), span (wave +
// 7919 it) mod spans, into LDS through the DMA unit (one span in flight per
// wave) or into registers.
template <int U, bool DMA>
__global__ __launch_bounds__(kThreads) void reread_kernel(const char* __restrict__ buf, int64_t spans, int iters,
                                                          uint32_t key, uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) char ring[kThreads / 64][U * 1024];
  const int lane = threadIdx.x & 63, wid = threadIdx.x / 64;
  const int64_t wave = int64_t(blockIdx.x) * (kThreads / 64) + wid;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
    const char* base = buf + ((wave + int64_t(it) * 7919) % spans) * U * 1024;
    if constexpr (DMA) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < U; ++u)
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) const void*)(base + u * 1024 + lane * 16),
                                         (__attribute__((address_space(3))) void*)(&ring[wid][u * 1024]), 16, 0, 0);
    } else {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const u32x4*>(base + u * 1024 + lane * 16);
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u];
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if constexpr (DMA) r ^= *reinterpret_cast<const uint32_t*>(&ring[wid][lane * 16]);
  if (r == key) sink[0] = r;
}

// Back-to-back MFMAs on register operands, NACC independent accumulators
// per wave, `iters` rounds; the accumulators are stored only if their sum
// equals `key`.
template <int NACC>
__global__ __launch_bounds__(kThreads) void mfma_bf16_kernel(int iters, float key, float* __restrict__ sink) {
  v8bf a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __bf16(float((threadIdx.x + i) & 7) * 0.125f);
    b[i] = __bf16(float((threadIdx.x * 3 + i) & 7) * 0.0625f);
  }
  v16f acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = v16f{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (s == key) sink[threadIdx.x] = s;
}

template <int NACC>
__global__ __launch_bounds__(kThreads) void mfma_i8_kernel(int iters, int key, int* __restrict__ sink) {
  v4i a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = int(0x01010101u * ((threadIdx.x + i) & 3));
    b[i] = int(0x01010101u * ((threadIdx.x * 3 + i) & 3));
  }
  v16i acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = v16i{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
  int s = 0;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (s == key) sink[threadIdx.x] = s;
}

template <int NACC>
__global__ __launch_bounds__(kThreads) void mfma_fp8_kernel(int iters, float key, float* __restrict__ sink) {
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = int(0x38383838u + ((threadIdx.x + i) & 3));   // E4M3 codes near 1.0
    b[i] = int(0x30303030u + ((threadIdx.x * 3 + i) & 3));
  }
  v16f acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = v16f{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < NACC; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 127);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (s == key) sink[threadIdx.x] = s;
}

constexpr int kNacc = 4;

}  // namespace

extern "C" {

int qlinear_ceiling_stream_read(const void* buf, int64_t bytes, int span_kib, int64_t blocks, void* sink,
                                void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || blocks < 1 || blocks > (int64_t(1) << 31) - 1 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return 1;
  auto s = static_cast<hipStream_t>(stream);
  const dim3 g{unsigned(blocks), 1, 1}, b{unsigned(kThreads), 1, 1};
  auto* p = static_cast<const u32x4*>(buf);
  auto* k = static_cast<uint32_t*>(sink);
  switch (span_kib) {
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, g, b, 0, s, p, bytes / 16, 0x9E3779B9u, k); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, g, b, 0, s, p, bytes / 16, 0x9E3779B9u, k); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, g, b, 0, s, p, bytes / 16, 0x9E3779B9u, k); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int qlinear_ceiling_stream_dma(const void* buf, int64_t bytes, int span_kib, int64_t blocks, void* sink,
                               void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || blocks < 1 || blocks > (int64_t(1) << 31) - 1 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return 1;
  auto s = static_cast<hipStream_t>(stream);
  const dim3 g{unsigned(blocks), 1, 1}, b{unsigned(kThreads), 1, 1};
  auto* p = static_cast<const char*>(buf);
  auto* k = static_cast<uint32_t*>(sink);
  switch (span_kib) {
    case 4: hipLaunchKernelGGL(stream_dma_kernel<4>, g, b, 0, s, p, bytes / 16, 0x9E3779B9u, k); break;
    case 8: hipLaunchKernelGGL(stream_dma_kernel<8>, g, b, 0, s, p, bytes / 16, 0x9E3779B9u, k); break;
    case 16: hipLaunchKernelGGL(stream_dma_kernel<16>, g, b, 0, s, p, bytes / 16, 0x9E3779B9u, k); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int qlinear_ceiling_reread(const void* buf, int64_t bytes, int dma, int64_t blocks, int iters, void* sink,
                           void* stream) {
  constexpr int U = 8;
  const int64_t spans = bytes / (U * 1024);
  if (!buf || !sink || spans < 1 || blocks < 1 || blocks > (int64_t(1) << 31) - 1 || iters < 1 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return 1;
  auto s = static_cast<hipStream_t>(stream);
  const dim3 g{unsigned(blocks), 1, 1}, b{unsigned(kThreads), 1, 1};
  auto* p = static_cast<const char*>(buf);
  auto* k = static_cast<uint32_t*>(sink);
  if (dma) hipLaunchKernelGGL((reread_kernel<U, true>), g, b, 0, s, p, spans, iters, 0x9E3779B9u, k);
  else hipLaunchKernelGGL((reread_kernel<U, false>), g, b, 0, s, p, spans, iters, 0x9E3779B9u, k);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// dtype: 0 bf16 (32x32x16), 1 int8 (32x32x32), 2 fp8 (32x32x64 f8f6f4).
// sink: device memory of at least 256 * 4 bytes.
int qlinear_ceiling_mfma(int dtype, int64_t blocks, int iters, void* sink, void* stream) {
  if (!sink || blocks < 1 || blocks > 65535 * 64 || iters < 1 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return 1;
  auto s = static_cast<hipStream_t>(stream);
  const dim3 g{unsigned(blocks), 1, 1}, b{unsigned(kThreads), 1, 1};
  switch (dtype) {
    case 0: hipLaunchKernelGGL(mfma_bf16_kernel<kNacc>, g, b, 0, s, iters, -1.f, static_cast<float*>(sink)); break;
    case 1: hipLaunchKernelGGL(mfma_i8_kernel<kNacc>, g, b, 0, s, iters, -7, static_cast<int*>(sink)); break;
    case 2: hipLaunchKernelGGL(mfma_fp8_kernel<kNacc>, g, b, 0, s, iters, -1.f, static_cast<float*>(sink)); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Operations one wave's round of qlinear_ceiling_mfma performs (2 M N K per
// instruction times the accumulators).
int64_t qlinear_ceiling_mfma_ops_per_wave_round(int dtype) {
  switch (dtype) {
    case 0: return int64_t(kNacc) * 2 * 32 * 32 * 16;
    case 1: return int64_t(kNacc) * 2 * 32 * 32 * 32;
    case 2: return int64_t(kNacc) * 2 * 32 * 32 * 64;
    default: return 0;
  }
}

}  // extern "C"
