// Device-side building blocks shared by the libqlinear kernels (gfx950 only):
// storage-format decoders, the float32 -> bfloat16 output rounding, the
// wave64 reduction and the vector types the matrix-core builtins take.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epilogue.hpp"

namespace qlinear {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- loads

// 16-byte global load.  The pointer must be 16-byte aligned.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 16-byte streaming load: the weight is read exactly once per launch, so it
// is marked non-temporal to keep it from displacing the reused activation.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------- decoders

// Four float8_e4m3fn bytes (byte i = element i) -> four floats, exact.  The
// gfx950 conversion decodes the OCP E4M3 "FN" encoding; the exhaustive
// 256-code materialisation test checks it against the CPU decoder.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float (&o)[4]) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);  // bytes 0, 1
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);   // bytes 2, 3
  o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
}

// One float8_e4m3fn byte (in bits 0..7) -> float, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(b, false)[0];
}

// Two float8_e4m3fn bytes (word `hi` of w) -> two packed bfloat16, exact:
// every E4M3 value has at most 4 significant bits and lies inside the
// bfloat16 exponent range, so the conversion (scale 1) never rounds.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  v2bf r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight float8_e4m3fn bytes -> eight bfloat16 in the matrix-core operand type.
__device__ __forceinline__ v8bf e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r.x = e4m3x2_to_bf16x2<false>(w0);
  r.y = e4m3x2_to_bf16x2<true>(w0);
  r.z = e4m3x2_to_bf16x2<false>(w1);
  r.w = e4m3x2_to_bf16x2<true>(w1);
  return __builtin_bit_cast(v8bf, r);
}

// Two E2M1 codes (byte BYTE of w; the low nibble is the even element) ->
// two floats, exact.  The gfx950 conversion takes a float scale but applies
// only its power-of-two part (the MX scale convention), so it is called with
// scale 1 and an E4M3 block scale is multiplied in afterwards.
template <int BYTE>
__device__ __forceinline__ void e2m1x2_to_f32(uint32_t w, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, BYTE);
  lo = r[0];
  hi = r[1];
}

// Two E2M1 codes times the E4M3 block scale s -> two floats, exact: every
// E2M1 x E4M3 product has at most 5 significant bits, far inside float32.
template <int BYTE>
__device__ __forceinline__ void e2m1x2_scaled_f32(uint32_t w, float s, float& lo, float& hi) {
  e2m1x2_to_f32<BYTE>(w, lo, hi);
  lo *= s;
  hi *= s;
}

// A 32-bit word as two packed bfloat16.  Taking the word by value matters:
// bit-casting a vector element (v.y) in place reads the vector's first
// element with this compiler.
__device__ __forceinline__ v2bf as_bf16x2(uint32_t v) { return __builtin_bit_cast(v2bf, v); }

// Eight E2M1 codes (the nibbles of w, the low nibble of each byte first) ->
// four packed bfloat16 pairs, exact (conversion scale 1; every E2M1 value is
// a bfloat16).
__device__ __forceinline__ void e2m1x8_to_bf16x8(uint32_t w, v2bf (&p)[4]) {
  p[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  p[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  p[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  p[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
}

// Two floats that are exactly representable in bfloat16 -> packed bfloat16
// (the upper halves; no rounding is needed).
__device__ __forceinline__ uint32_t pack_exact_bf16x2(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Two E2M1 codes times the E4M3 block scale s -> two packed bfloat16, exact
// (the products also lie inside the bfloat16 exponent range).  The
// exhaustive NVFP4 dequantisation test checks this decoder against the CPU.
template <int BYTE>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w, float s) {
  float lo, hi;
  e2m1x2_scaled_f32<BYTE>(w, s, lo, hi);
  return pack_exact_bf16x2(lo, hi);
}

// Packed bfloat16 pair -> floats (exact: bfloat16 is the top half of binary32).
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// float32 -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ---------------------------------------------------------------- epilogue store

// out[i] = round(alpha * acc) in the output type (0 = float32, 1 = bfloat16).
__device__ __forceinline__ void store_out(void* out, int64_t i, float acc, float alpha, int out_bf16) {
  const float v = acc * alpha;
  if (out_bf16) reinterpret_cast<uint16_t*>(out)[i] = f32_to_bf16(v);
  else reinterpret_cast<float*>(out)[i] = v;
}

// ---------------------------------------------------------------- fused epilogue

// Fused epilogue (the steps are listed at Epilogue) of output element (m, n).
// x * sigmoid(z), accurate to a few float32 ulps of the result at every z:
// e = exp(-|z|) never overflows, and neither branch subtracts nearly equal
// numbers (for z < 0, x e / (1 + e) rather than x / (1 + e^-z)).
__device__ __forceinline__ float mul_sigmoid(float x, float z) {
  const float e = expf(-fabsf(z));
  const float d = 1.f + e;
  return z >= 0.f ? x / d : x * e / d;
}

__device__ __forceinline__ float epi_apply(const Epilogue& e, float v, int64_t m, int64_t n) {
  if (e.row_scale) v *= e.row_scale[m];
  if (e.col_scale) v *= e.col_scale[n];
  if (e.bias) v += bf16_to_f32(e.bias[n]);
  if (e.act == 1) {
    v = v > 0.f ? v : 0.f;
  } else if (e.act == 2) {
    v = mul_sigmoid(v, v);  // SiLU
  } else if (e.act == 3) {
    // GELU, tanh form: 0.5 v (1 + tanh(u)) = v sigmoid(2 u), which keeps its
    // relative accuracy where 1 + tanh(u) would cancel (v below about -4).
    const float u = 0.7978845608028654f * (v + 0.044715f * v * v * v);
    v = mul_sigmoid(v, 2.f * u);
  }
  if (e.residual) {
    const int64_t i = m * e.ld + n;
    v += e.res_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(e.residual)[i])
                    : reinterpret_cast<const float*>(e.residual)[i];
  }
  return v;
}

// out[m * N + n] = round(epilogue(alpha * acc)) in the output type.
__device__ __forceinline__ void store_epi(void* out, int64_t m, int64_t n, int64_t N, float acc, float alpha,
                                          int out_bf16, const Epilogue& epi) {
  float v = acc * alpha;
  if (epi.on) v = epi_apply(epi, v, m, n);
  const int64_t i = m * N + n;
  if (out_bf16) reinterpret_cast<uint16_t*>(out)[i] = f32_to_bf16(v);
  else reinterpret_cast<float*>(out)[i] = v;
}

// store_epi when the kernel instance carries the fused epilogue (FUSED),
// else the plain store: kernels whose registers the epilogue code would
// raise come in both forms.
template <bool FUSED>
__device__ __forceinline__ void store_maybe_epi(void* out, int64_t m, int64_t n, int64_t N, float acc, float alpha,
                                                int out_bf16, const Epilogue& epi) {
  if constexpr (FUSED) store_epi(out, m, n, N, acc, alpha, out_bf16, epi);
  else store_out(out, m * N + n, acc, alpha, out_bf16);
}


// ---------------------------------------------------------------- LDS DMA and waits

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// 16 bytes per lane from global memory straight into LDS: lane i's bytes
// land at lds + 16 i (lds is uniform over the wave).
__device__ __forceinline__ void dma16(const char* g, char* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds, 16, 0, 0);
}

// dma16 with the non-temporal hint (cache-policy bit 1, "nt"), for data that
// is read once, as the GEMV's weight loads are.
__device__ __forceinline__ void dma16_nt(const char* g, char* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds, 16, 0, 2);
}

// Wait until at most N vector-memory operations of this wave are
// outstanding.  The memory clobber keeps the compiler from moving LDS
// accesses across the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier without the release/acquire fences of __syncthreads():
// the fences would wait for every outstanding vector-memory operation,
// including the strips still in flight.  Callers wait for what must be
// complete (their share of the next strip, their own LDS reads) first; the
// asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- wave reduction

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
  return v + __int_as_float(moved);
}

// Sum over the 64 lanes of a wave; the total is returned in every lane.
// Steps: pairs and quads inside each row of 16 (quad_perm), the two halves
// of the row (row_half_mirror), the row (row_mirror), then the four rows
// through row_bcast:15 / row_bcast:31, which leaves the total in lane 63.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);          // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);          // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);         // row_half_mirror
  v = dpp_add<0x140>(v);         // row_mirror
  v = dpp_add<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

}  // namespace qlinear
