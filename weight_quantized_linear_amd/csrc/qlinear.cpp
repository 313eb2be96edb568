// The C ABI of libqlinear: argument validation, the gfx950 device check and
// the choice of kernel.  Declarations and the contract of every call are in
// include/qlinear.h.
#include "qlinear.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <limits>
#include <mutex>

#include "launch.hpp"

namespace {

using namespace qlinear;

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  std::atomic<int> state{0};  // 0 unknown, 1 gfx950, 2 other arch, 3 query failed
  int num_cus = 0;
};
DeviceInfo g_devices[kMaxDevices];
std::mutex g_device_mutex;

// Status of the current device, cached per device index; fills num_cus.
int current_device(int* num_cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLINEAR_ERR_DEVICE;
  DeviceInfo& d = g_devices[dev];
  int st = d.state.load(std::memory_order_acquire);
  if (st == 0) {
    std::lock_guard<std::mutex> lock(g_device_mutex);
    st = d.state.load(std::memory_order_relaxed);
    if (st == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        st = 3;
      } else {
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        d.num_cus = prop.multiProcessorCount;
      }
      d.state.store(st, std::memory_order_release);
    }
  }
  if (st == 3) return QLINEAR_ERR_DEVICE;
  if (st == 2) return QLINEAR_ERR_UNSUPPORTED;
  *num_cus = d.num_cus > 0 ? d.num_cus : 256;
  return QLINEAR_OK;
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// n1 * n2 (* n3) must stay addressable; all factors are already > 0.
bool fits(int64_t a, int64_t b, int64_t c = 1) {
  const int64_t lim = std::numeric_limits<int64_t>::max() / 8;
  if (a > lim / b) return false;
  const int64_t ab = a * b;
  return ab <= lim / c;
}

int float_out_ok(int out_dtype) { return out_dtype == QLINEAR_F32 || out_dtype == QLINEAR_BF16; }

size_t out_size(int out_dtype) { return out_dtype == QLINEAR_BF16 ? 2 : 4; }

int finish(hipError_t e) { return e == hipSuccess ? QLINEAR_OK : QLINEAR_ERR_LAUNCH; }

// Validates a caller's epilogue for an [M, N] output and converts it (null:
// no epilogue).  The residual may be the output itself (same type, ld = N).
int to_epilogue(const qlinear_epilogue* e, int64_t M, int64_t N, Epilogue* out) {
  *out = Epilogue{};
  if (!e) return QLINEAR_OK;
  if (e->activation < QLINEAR_ACT_NONE || e->activation > QLINEAR_ACT_GELU_TANH) return QLINEAR_ERR_INVALID_ARG;
  if ((e->row_scale && !aligned(e->row_scale, 4)) || (e->col_scale && !aligned(e->col_scale, 4)) ||
      (e->bias && !aligned(e->bias, 2)))
    return QLINEAR_ERR_INVALID_ARG;
  if (e->residual) {
    if (e->residual_dtype != QLINEAR_F32 && e->residual_dtype != QLINEAR_BF16) return QLINEAR_ERR_INVALID_ARG;
    if (e->residual_ld < N || !aligned(e->residual, out_size(e->residual_dtype)) || !fits(M, e->residual_ld))
      return QLINEAR_ERR_INVALID_ARG;
  }
  out->row_scale = e->row_scale;
  out->col_scale = e->col_scale;
  out->bias = static_cast<const uint16_t*>(e->bias);
  out->residual = e->residual;
  out->ld = e->residual ? e->residual_ld : 0;
  out->act = e->activation;
  out->res_bf16 = e->residual_dtype == QLINEAR_BF16;
  out->on = e->row_scale || e->col_scale || e->bias || e->residual || e->activation != QLINEAR_ACT_NONE;
  return QLINEAR_OK;
}

// A caller's split-K workspace: NULL (with 0 bytes) for none, else at least
// 16-byte aligned device memory of workspace_bytes >= 0 bytes.
int check_workspace(const void* ws, int64_t ws_bytes) {
  if (ws_bytes < 0 || (!ws && ws_bytes != 0) || (ws && !aligned(ws, 16))) return QLINEAR_ERR_INVALID_ARG;
  return QLINEAR_OK;
}

// The FP8 kernel family that a call takes: `path` if forced, else the
// automatic choice, which depends on the shape, the operands' alignment and
// whether a workspace of at least `ws_need` bytes is given (and on nothing
// else, so that a call is reproducible from its arguments).
int fp8_choose(int path, int64_t M, int64_t N, int64_t K, bool wide, bool splitk_ok) {
  if (path != QLINEAR_PATH_AUTO) return path;
  // Measured on the decode shapes: the vector-ALU GEMV wins for M <= 2
  // below 65536 output features and for M <= 4 on small weights; the
  // matrix-core skinny kernels win above that (for 3 <= M <= 4 from 8192
  // output features or a K of 8192 when the activation-in-LDS kernel
  // applies, and for M = 4 from 4096 output features where the streaming
  // kernel takes the shape) and for 5 <= M <= 16; beyond 16 rows the
  // LDS-tiled GEMM.
  const bool big = N >= 65536 || (M >= 3 && (N >= 8192 || K >= 8192) && fp8_skinny_xlds_supported(M, N, K)) ||
                   (M == 4 && fp8_skinny_stream_wins(M, N, K) && (K == 1024 || K == 2048 || K == 3072 || K == 4096));
  // Split-K needs the caller's workspace.  Where K is made of 2048-value
  // slices (K >= 8192) and there are fewer than 65536 output features, its
  // streaming form wins from M = 3 (N = 4096, K = 14336: M = 4 14.8 against
  // 17.2 us for the 4x4x4 skinny kernel, M = 8 15.4 against 18.5; N = K =
  // 14336, M = 8: 40.1 against 51.7) and at M = 2 from 8192 output features
  // (N = K = 14336: 37.2 against 47.2 us for the GEMV; at N = 4096 the GEMV
  // keeps 12.6 against 14.3); for 9 <= M <= 16 the split-K skinny kernel also
  // wins at other long K (M = 16, N = 4096, K = 14336: 19.2 against 23.1 us).
  const bool split_long = splitk_ok && wide && K >= 8192 && N < 65536;
  if (M == 1) return QLINEAR_PATH_GEMV;
  if (M <= 4) {
    if ((M >= 3 || N >= 8192) && split_long && K % 2048 == 0) return QLINEAR_PATH_SPLITK;
    return (wide && big) ? QLINEAR_PATH_SKINNY : QLINEAR_PATH_GEMV;
  }
  if (M <= 16 && wide)
    return (split_long && (K % 2048 == 0 || (M > 8 && K % 64 == 0))) ? QLINEAR_PATH_SPLITK : QLINEAR_PATH_SKINNY;
  return QLINEAR_PATH_TILED;
}

int nvfp4_choose(int path, int64_t M) {
  if (path != QLINEAR_PATH_AUTO) return path;
  return M <= 4 ? QLINEAR_PATH_GEMV : QLINEAR_PATH_TILED;
}

int bf16_choose(int path, int64_t M, bool wide) {
  if (path != QLINEAR_PATH_AUTO) return path;
  if (M <= 4) return QLINEAR_PATH_GEMV;
  if (M <= 16 && wide) return QLINEAR_PATH_SKINNY;
  return QLINEAR_PATH_TILED;
}

}  // namespace

namespace qlinear {

int fp8_gemm_impl(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                  float alpha, int path, void* ws, int64_t ws_bytes, void* stream,
                  const qlinear_epilogue* epilogue = nullptr) {
  if (!w || !x || !out) return QLINEAR_ERR_INVALID_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || !fits(N, K) || !fits(M, K) || !fits(M, N))
    return QLINEAR_ERR_INVALID_ARG;
  if (!float_out_ok(out_dtype)) return QLINEAR_ERR_INVALID_ARG;
  if (!aligned(x, 2) || !aligned(out, out_size(out_dtype))) return QLINEAR_ERR_INVALID_ARG;
  if (int st = check_workspace(ws, ws_bytes)) return st;
  const bool wide = K % 16 == 0 && aligned(w, 16) && aligned(x, 16);
  switch (path) {
    case QLINEAR_PATH_AUTO:
    case QLINEAR_PATH_TILED:
      break;
    case QLINEAR_PATH_GEMV:
      if (M > 4) return QLINEAR_ERR_INVALID_ARG;
      break;
    case QLINEAR_PATH_SKINNY:
      if (M > 16 || !wide) return QLINEAR_ERR_INVALID_ARG;
      break;
    case QLINEAR_PATH_SPLITK:
      if (M > 16 || !wide || K % 64 != 0) return QLINEAR_ERR_INVALID_ARG;
      break;
    default:
      return QLINEAR_ERR_INVALID_ARG;
  }
  Epilogue epi;
  if (int st = to_epilogue(epilogue, M, N, &epi)) return st;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  const size_t splitk_need = fp8_skinny_splitk_ws_bytes(M, N, K, num_cus);
  const bool splitk_ok = ws && splitk_need > 0 && splitk_need <= size_t(ws_bytes);
  path = fp8_choose(path, M, N, K, wide, splitk_ok);
  // Forced split-K with fewer than two K slices or planes beyond the workspace.
  if (path == QLINEAR_PATH_SPLITK && !splitk_ok) return QLINEAR_ERR_UNSUPPORTED;
  auto s = static_cast<hipStream_t>(stream);
  auto* wp = static_cast<const uint8_t*>(w);
  auto* xp = static_cast<const uint16_t*>(x);
  auto* wsp = static_cast<float*>(ws);
  const int bf16 = out_dtype == QLINEAR_BF16;
  if (path == QLINEAR_PATH_SPLITK)
    return finish(launch_fp8_skinny_splitk(wp, xp, out, bf16, M, N, K, alpha, num_cus, wsp, size_t(ws_bytes), s, epi));
  if (path == QLINEAR_PATH_GEMV)
    return finish(launch_fp8_gemv(wp, xp, out, bf16, M, N, K, alpha, num_cus, s, epi));
  if (path == QLINEAR_PATH_SKINNY)
    return finish(launch_fp8_skinny(wp, xp, out, bf16, M, N, K, alpha, num_cus, s, epi));
  return finish(launch_fp8_tiled(wp, xp, out, bf16, M, N, K, alpha, num_cus, wsp, size_t(ws_bytes), s, epi));
}

int fp8_gemm_ws_need(int path, int64_t M, int64_t N, int64_t K, int num_cus, int64_t* bytes) {
  *bytes = 0;
  if (M <= 0 || N <= 0 || K <= 0 || !fits(N, K) || !fits(M, K) || !fits(M, N)) return QLINEAR_ERR_INVALID_ARG;
  const size_t splitk = fp8_skinny_splitk_ws_bytes(M, N, K, num_cus);
  path = fp8_choose(path, M, N, K, K % 16 == 0, splitk > 0);
  if (path == QLINEAR_PATH_SPLITK) *bytes = int64_t(splitk);
  else if (path == QLINEAR_PATH_TILED && K % 64 == 0) *bytes = int64_t(fp8_gemm_lds_ws_bytes(M, N, K, num_cus));
  return QLINEAR_OK;
}

}  // namespace qlinear

namespace {

int nvfp4_gemm_impl(const void* wp, const void* wsc, const void* x, void* out, int out_dtype, int64_t M, int64_t N,
                    int64_t K, float alpha, int path, void* ws, int64_t ws_bytes, void* stream,
                    const qlinear_epilogue* epilogue = nullptr) {
  if (!wp || !wsc || !x || !out) return QLINEAR_ERR_INVALID_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0 || !fits(N, K) || !fits(M, K) || !fits(M, N))
    return QLINEAR_ERR_INVALID_ARG;
  if (!float_out_ok(out_dtype) || !aligned(x, 2) || !aligned(out, out_size(out_dtype)))
    return QLINEAR_ERR_INVALID_ARG;
  if (int st = check_workspace(ws, ws_bytes)) return st;
  path = nvfp4_choose(path, M);
  if (path == QLINEAR_PATH_GEMV) {
    if (M > 4) return QLINEAR_ERR_INVALID_ARG;
  } else if (path != QLINEAR_PATH_TILED) {
    return QLINEAR_ERR_INVALID_ARG;
  }
  Epilogue epi;
  if (int st = to_epilogue(epilogue, M, N, &epi)) return st;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  auto s = static_cast<hipStream_t>(stream);
  auto* p = static_cast<const uint8_t*>(wp);
  auto* sc = static_cast<const uint8_t*>(wsc);
  auto* xp = static_cast<const uint16_t*>(x);
  const int bf16 = out_dtype == QLINEAR_BF16;
  if (path == QLINEAR_PATH_GEMV)
    return finish(launch_nvfp4_gemv(p, sc, xp, out, bf16, M, N, K, alpha, num_cus, s, epi));
  return finish(launch_nvfp4_tiled(p, sc, xp, out, bf16, M, N, K, alpha, num_cus, static_cast<float*>(ws),
                                   size_t(ws_bytes), s, epi));
}

int bf16_gemm_impl(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                   float alpha, int path, void* ws, int64_t ws_bytes, void* stream,
                   const qlinear_epilogue* epilogue = nullptr) {
  if (!w || !x || !out) return QLINEAR_ERR_INVALID_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || !fits(N, K) || !fits(M, K) || !fits(M, N))
    return QLINEAR_ERR_INVALID_ARG;
  if (!float_out_ok(out_dtype)) return QLINEAR_ERR_INVALID_ARG;
  if (!aligned(w, 2) || !aligned(x, 2) || !aligned(out, out_size(out_dtype))) return QLINEAR_ERR_INVALID_ARG;
  if (int st = check_workspace(ws, ws_bytes)) return st;
  const bool wide = bf16_wide(w, x, K);
  path = bf16_choose(path, M, wide);
  switch (path) {
    case QLINEAR_PATH_GEMV:
      if (M > 4) return QLINEAR_ERR_INVALID_ARG;
      break;
    case QLINEAR_PATH_SKINNY:
      if (M > 16 || !wide) return QLINEAR_ERR_INVALID_ARG;
      break;
    case QLINEAR_PATH_TILED:
      break;
    default:
      return QLINEAR_ERR_INVALID_ARG;
  }
  Epilogue epi;
  if (int st = to_epilogue(epilogue, M, N, &epi)) return st;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  auto s = static_cast<hipStream_t>(stream);
  auto* wp = static_cast<const uint16_t*>(w);
  auto* xp = static_cast<const uint16_t*>(x);
  const int bf16 = out_dtype == QLINEAR_BF16;
  if (path == QLINEAR_PATH_GEMV)
    return finish(launch_bf16_gemv(wp, xp, out, bf16, M, N, K, alpha, num_cus, s, epi));
  if (path == QLINEAR_PATH_SKINNY)
    return finish(launch_bf16_skinny(wp, xp, out, bf16, M, N, K, alpha, num_cus, s, epi));
  return finish(launch_bf16_tiled(wp, xp, out, bf16, M, N, K, alpha, num_cus, static_cast<float*>(ws),
                                  size_t(ws_bytes), s, epi));
}

}  // namespace

extern "C" {

int qlinear_abi_version(void) { return QLINEAR_ABI_VERSION; }

const char* qlinear_status_string(int status) {
  switch (status) {
    case QLINEAR_OK: return "ok";
    case QLINEAR_ERR_INVALID_ARG: return "invalid argument";
    case QLINEAR_ERR_UNSUPPORTED: return "unsupported device or configuration";
    case QLINEAR_ERR_DEVICE: return "no usable HIP device";
    case QLINEAR_ERR_LAUNCH: return "kernel launch failed";
    case QLINEAR_ERR_SCRATCH_LIMIT: return "shape needs more split-K scratch than the library's fixed buffer";
    default: return "unknown status";
  }
}

int qlinear_fp8_gemv(const void* w, const void* x, void* out, int out_dtype, int64_t N, int64_t K,
                     float alpha, void* stream) {
  return fp8_gemm_impl(w, x, out, out_dtype, 1, N, K, alpha, QLINEAR_PATH_GEMV, nullptr, 0, stream);
}

int qlinear_fp8_gemm(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N,
                     int64_t K, float alpha, void* stream) {
  return fp8_gemm_impl(w, x, out, out_dtype, M, N, K, alpha, QLINEAR_PATH_AUTO, nullptr, 0, stream);
}

int qlinear_fp8_gemm_path(const void* w, const void* x, void* out, int out_dtype, int64_t M,
                          int64_t N, int64_t K, float alpha, int path, void* stream) {
  return fp8_gemm_impl(w, x, out, out_dtype, M, N, K, alpha, path, nullptr, 0, stream);
}

int qlinear_fp8_materialize(const void* w, void* out, int out_dtype, int64_t N, int64_t K,
                            void* stream) {
  if (!w || !out || N <= 0 || K <= 0 || !fits(N, K) || !float_out_ok(out_dtype))
    return QLINEAR_ERR_INVALID_ARG;
  if (!aligned(out, out_size(out_dtype))) return QLINEAR_ERR_INVALID_ARG;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  return finish(launch_fp8_materialize(static_cast<const uint8_t*>(w), out,
                                       out_dtype == QLINEAR_BF16, N * K,
                                       static_cast<hipStream_t>(stream)));
}

int qlinear_fp8_grouped_gemm(const void* w, const void* x, const uint32_t* a_offsets,
                             const int32_t* expert_ids, void* out, int out_dtype, int64_t num_groups,
                             int64_t max_tokens_per_group, int64_t num_experts, int64_t T, int64_t N,
                             int64_t K, void* stream) {
  return qlinear_fp8_grouped_gemm_scaled(w, x, a_offsets, expert_ids, nullptr, out, out_dtype, num_groups,
                                         max_tokens_per_group, num_experts, T, N, K, stream);
}

int qlinear_fp8_grouped_gemm_scaled(const void* w, const void* x, const uint32_t* a_offsets,
                                    const int32_t* expert_ids, const float* expert_scale, void* out, int out_dtype,
                                    int64_t num_groups, int64_t max_tokens_per_group, int64_t num_experts, int64_t T,
                                    int64_t N, int64_t K, void* stream) {
  if (!w || !x || !a_offsets || !expert_ids || !out) return QLINEAR_ERR_INVALID_ARG;
  if (expert_scale && !aligned(expert_scale, 4)) return QLINEAR_ERR_INVALID_ARG;
  if (num_groups <= 0 || num_groups > 65535 || max_tokens_per_group < 0 || num_experts <= 0 || T <= 0 ||
      N <= 0 || K <= 0)
    return QLINEAR_ERR_INVALID_ARG;
  if (!fits(num_experts, N, K) || !fits(T, K) || !fits(T, N)) return QLINEAR_ERR_INVALID_ARG;
  if (!float_out_ok(out_dtype) || !aligned(x, 2) || !aligned(out, out_size(out_dtype)) ||
      !aligned(a_offsets, 4) || !aligned(expert_ids, 4))
    return QLINEAR_ERR_INVALID_ARG;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  return finish(launch_fp8_grouped(static_cast<const uint8_t*>(w), static_cast<const uint16_t*>(x),
                                   a_offsets, expert_ids, out, out_dtype == QLINEAR_BF16, num_groups,
                                   max_tokens_per_group, num_experts, T, N, K, num_cus,
                                   static_cast<hipStream_t>(stream), expert_scale));
}

int qlinear_fp8_quantize_act(const void* x, void* q, float input_scale, int64_t M, int64_t K, void* stream) {
  if (!x || !q || M <= 0 || K <= 0 || !fits(M, K) || !aligned(x, 2)) return QLINEAR_ERR_INVALID_ARG;
  if (!(input_scale > 0.f) || !(input_scale <= std::numeric_limits<float>::max())) return QLINEAR_ERR_INVALID_ARG;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  return finish(launch_fp8_quantize_act(static_cast<const uint16_t*>(x), static_cast<uint8_t*>(q), input_scale, M, K,
                                        num_cus, static_cast<hipStream_t>(stream)));
}

int qlinear_fp8_w8a8_gemm(const void* xq, const void* w, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                          float alpha, void* stream) {
  if (!xq || !w || !out || M <= 0 || N <= 0 || K <= 0 || !fits(M, K) || !fits(N, K) || !fits(M, N))
    return QLINEAR_ERR_INVALID_ARG;
  if (!float_out_ok(out_dtype) || !aligned(out, out_size(out_dtype))) return QLINEAR_ERR_INVALID_ARG;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  return finish(launch_fp8_w8a8_gemm(static_cast<const uint8_t*>(xq), static_cast<const uint8_t*>(w), out,
                                     out_dtype == QLINEAR_BF16, M, N, K, alpha, num_cus,
                                     static_cast<hipStream_t>(stream)));
}

int qlinear_nvfp4_grouped_gemm(const void* w_packed, const void* w_scale, const void* x, const uint32_t* a_offsets,
                               const int32_t* expert_ids, void* out, int out_dtype, int64_t num_groups,
                               int64_t max_tokens_per_group, int64_t num_experts, int64_t T, int64_t N, int64_t K,
                               void* stream) {
  return qlinear_nvfp4_grouped_gemm_scaled(w_packed, w_scale, x, a_offsets, expert_ids, nullptr, out, out_dtype,
                                           num_groups, max_tokens_per_group, num_experts, T, N, K, stream);
}

int qlinear_nvfp4_grouped_gemm_scaled(const void* w_packed, const void* w_scale, const void* x,
                                      const uint32_t* a_offsets, const int32_t* expert_ids, const float* expert_scale,
                                      void* out, int out_dtype, int64_t num_groups, int64_t max_tokens_per_group,
                                      int64_t num_experts, int64_t T, int64_t N, int64_t K, void* stream) {
  if (!w_packed || !w_scale || !x || !a_offsets || !expert_ids || !out) return QLINEAR_ERR_INVALID_ARG;
  if (expert_scale && !aligned(expert_scale, 4)) return QLINEAR_ERR_INVALID_ARG;
  if (num_groups <= 0 || num_groups > 65535 || max_tokens_per_group < 0 || num_experts <= 0 || T <= 0 ||
      N <= 0 || K <= 0 || K % 16 != 0)
    return QLINEAR_ERR_INVALID_ARG;
  if (!fits(num_experts, N, K) || !fits(T, K) || !fits(T, N)) return QLINEAR_ERR_INVALID_ARG;
  if (!float_out_ok(out_dtype) || !aligned(x, 2) || !aligned(out, out_size(out_dtype)) ||
      !aligned(a_offsets, 4) || !aligned(expert_ids, 4))
    return QLINEAR_ERR_INVALID_ARG;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  return finish(launch_nvfp4_grouped(static_cast<const uint8_t*>(w_packed), static_cast<const uint8_t*>(w_scale),
                                     static_cast<const uint16_t*>(x), a_offsets, expert_ids, out,
                                     out_dtype == QLINEAR_BF16, num_groups, max_tokens_per_group, num_experts, T,
                                     N, K, num_cus, static_cast<hipStream_t>(stream), expert_scale));
}

int qlinear_nvfp4_gemm(const void* w_packed, const void* w_scale, const void* x, void* out, int out_dtype,
                       int64_t M, int64_t N, int64_t K, float alpha, void* stream) {
  return nvfp4_gemm_impl(w_packed, w_scale, x, out, out_dtype, M, N, K, alpha, QLINEAR_PATH_AUTO, nullptr, 0, stream);
}

int qlinear_nvfp4_gemm_path(const void* w_packed, const void* w_scale, const void* x, void* out,
                            int out_dtype, int64_t M, int64_t N, int64_t K, float alpha, int path,
                            void* stream) {
  return nvfp4_gemm_impl(w_packed, w_scale, x, out, out_dtype, M, N, K, alpha, path, nullptr, 0, stream);
}

int qlinear_nvfp4_dequant(const void* w_packed, const void* w_scale, void* out, int out_dtype, int64_t N,
                          int64_t K, void* stream) {
  if (!w_packed || !w_scale || !out || N <= 0 || K <= 0 || K % 16 != 0 || !fits(N, K) ||
      !float_out_ok(out_dtype) || !aligned(out, out_size(out_dtype)))
    return QLINEAR_ERR_INVALID_ARG;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  return finish(launch_nvfp4_dequant(static_cast<const uint8_t*>(w_packed), static_cast<const uint8_t*>(w_scale),
                                     out, out_dtype == QLINEAR_BF16, N, K, static_cast<hipStream_t>(stream)));
}

int qlinear_int8_quantize_act(const void* x, void* q, float* a_scale, int64_t M, int64_t K, void* stream) {
  if (!x || !q || !a_scale || M <= 0 || K <= 0 || !fits(M, K) || !aligned(x, 2) || !aligned(a_scale, 4))
    return QLINEAR_ERR_INVALID_ARG;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  return finish(launch_int8_quantize(static_cast<const uint16_t*>(x), static_cast<int8_t*>(q), a_scale, M, K,
                                     static_cast<hipStream_t>(stream)));
}

int qlinear_int8_gemm(const void* a, const void* b, const float* a_scale, const float* b_scale,
                      const void* bias, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                      void* stream) {
  if (!a || !b || !out || M <= 0 || N <= 0 || K <= 0 || K > 133144) return QLINEAR_ERR_INVALID_ARG;
  if (!fits(M, K) || !fits(N, K) || !fits(M, N)) return QLINEAR_ERR_INVALID_ARG;
  int mode;
  if (out_dtype == QLINEAR_F32) mode = 0;
  else if (out_dtype == QLINEAR_BF16) mode = 1;
  else if (out_dtype == QLINEAR_I32) mode = 2;
  else return QLINEAR_ERR_INVALID_ARG;
  if (mode != 2 && (!a_scale || !b_scale || !aligned(a_scale, 4) || !aligned(b_scale, 4)))
    return QLINEAR_ERR_INVALID_ARG;
  if (mode != 2 && bias && !aligned(bias, 2)) return QLINEAR_ERR_INVALID_ARG;
  if (!aligned(out, mode == 1 ? 2 : 4)) return QLINEAR_ERR_INVALID_ARG;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  return finish(launch_int8_gemm(static_cast<const int8_t*>(a), static_cast<const int8_t*>(b), a_scale, b_scale,
                                 mode == 2 ? nullptr : static_cast<const uint16_t*>(bias), out, mode, M, N, K,
                                 num_cus, static_cast<hipStream_t>(stream)));
}

int qlinear_bf16_gemm(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                      float alpha, void* stream) {
  return bf16_gemm_impl(w, x, out, out_dtype, M, N, K, alpha, QLINEAR_PATH_AUTO, nullptr, 0, stream);
}

int qlinear_bf16_gemm_path(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                           float alpha, int path, void* stream) {
  return bf16_gemm_impl(w, x, out, out_dtype, M, N, K, alpha, path, nullptr, 0, stream);
}

int qlinear_fp8_gemm_epilogue(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N,
                              int64_t K, float alpha, const qlinear_epilogue* epilogue, void* stream) {
  return fp8_gemm_impl(w, x, out, out_dtype, M, N, K, alpha, QLINEAR_PATH_AUTO, nullptr, 0, stream, epilogue);
}

int qlinear_fp8_gemm_epilogue_path(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N,
                                   int64_t K, float alpha, const qlinear_epilogue* epilogue, int path, void* stream) {
  return fp8_gemm_impl(w, x, out, out_dtype, M, N, K, alpha, path, nullptr, 0, stream, epilogue);
}

int qlinear_nvfp4_gemm_epilogue(const void* w_packed, const void* w_scale, const void* x, void* out, int out_dtype,
                                int64_t M, int64_t N, int64_t K, float alpha, const qlinear_epilogue* epilogue,
                                void* stream) {
  return nvfp4_gemm_impl(w_packed, w_scale, x, out, out_dtype, M, N, K, alpha, QLINEAR_PATH_AUTO, nullptr, 0, stream, epilogue);
}

int qlinear_bf16_gemm_epilogue(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N,
                               int64_t K, float alpha, const qlinear_epilogue* epilogue, void* stream) {
  return bf16_gemm_impl(w, x, out, out_dtype, M, N, K, alpha, QLINEAR_PATH_AUTO, nullptr, 0, stream, epilogue);
}

int qlinear_int8_grouped_gemm(const void* a, const void* b, const float* a_scale, const float* b_scale,
                              const void* bias, const uint32_t* a_offsets, const int32_t* expert_ids, void* out,
                              int out_dtype, int64_t num_groups, int64_t max_tokens_per_group, int64_t num_experts,
                              int64_t T, int64_t N, int64_t K, void* stream) {
  if (!a || !b || !a_offsets || !expert_ids || !out) return QLINEAR_ERR_INVALID_ARG;
  if (num_groups <= 0 || num_groups > 65535 || max_tokens_per_group < 0 || num_experts <= 0 || T <= 0 ||
      N <= 0 || K <= 0 || K > 133144)
    return QLINEAR_ERR_INVALID_ARG;
  if (!fits(num_experts, N, K) || !fits(T, K) || !fits(T, N)) return QLINEAR_ERR_INVALID_ARG;
  int mode;
  if (out_dtype == QLINEAR_F32) mode = 0;
  else if (out_dtype == QLINEAR_BF16) mode = 1;
  else if (out_dtype == QLINEAR_I32) mode = 2;
  else return QLINEAR_ERR_INVALID_ARG;
  if (mode != 2 && (!a_scale || !b_scale || !aligned(a_scale, 4) || !aligned(b_scale, 4)))
    return QLINEAR_ERR_INVALID_ARG;
  if (mode != 2 && bias && !aligned(bias, 2)) return QLINEAR_ERR_INVALID_ARG;
  if (!aligned(out, mode == 1 ? 2 : 4) || !aligned(a_offsets, 4) || !aligned(expert_ids, 4))
    return QLINEAR_ERR_INVALID_ARG;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  return finish(launch_int8_grouped(static_cast<const int8_t*>(a), static_cast<const int8_t*>(b),
                                    mode == 2 ? nullptr : a_scale, mode == 2 ? nullptr : b_scale,
                                    mode == 2 ? nullptr : static_cast<const uint16_t*>(bias), a_offsets, expert_ids,
                                    out, mode, num_groups, max_tokens_per_group, num_experts, T, N, K, num_cus,
                                    static_cast<hipStream_t>(stream)));
}

int qlinear_gemm_workspace_size(int weight_format, int path, int64_t M, int64_t N, int64_t K, int64_t* bytes) {
  if (!bytes) return QLINEAR_ERR_INVALID_ARG;
  *bytes = 0;
  if (M <= 0 || N <= 0 || K <= 0 || !fits(N, K) || !fits(M, K) || !fits(M, N)) return QLINEAR_ERR_INVALID_ARG;
  if (path < QLINEAR_PATH_AUTO || path > QLINEAR_PATH_SPLITK) return QLINEAR_ERR_INVALID_ARG;
  if (weight_format < QLINEAR_WEIGHT_FP8 || weight_format > QLINEAR_WEIGHT_BF16) return QLINEAR_ERR_INVALID_ARG;
  if (weight_format == QLINEAR_WEIGHT_NVFP4 && K % 16 != 0) return QLINEAR_ERR_INVALID_ARG;
  int num_cus = 0;
  if (int st = current_device(&num_cus)) return st;
  switch (weight_format) {
    case QLINEAR_WEIGHT_FP8:
      return fp8_gemm_ws_need(path, M, N, K, num_cus, bytes);
    case QLINEAR_WEIGHT_NVFP4:
      if (nvfp4_choose(path, M) == QLINEAR_PATH_TILED && K % 64 == 0)
        *bytes = int64_t(nvfp4_gemm_lds_ws_bytes(M, N, K, num_cus));
      return QLINEAR_OK;
    case QLINEAR_WEIGHT_BF16:
      if (bf16_choose(path, M, K % 8 == 0) == QLINEAR_PATH_TILED && K % 64 == 0)
        *bytes = int64_t(bf16_gemm_lds_ws_bytes(M, N, K, num_cus));
      return QLINEAR_OK;
    default:
      return QLINEAR_ERR_INVALID_ARG;
  }
}

int qlinear_fp8_gemm_ws(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                        float alpha, const qlinear_epilogue* epilogue, int path, void* workspace,
                        int64_t workspace_bytes, void* stream) {
  return fp8_gemm_impl(w, x, out, out_dtype, M, N, K, alpha, path, workspace, workspace_bytes, stream, epilogue);
}

int qlinear_nvfp4_gemm_ws(const void* w_packed, const void* w_scale, const void* x, void* out, int out_dtype,
                          int64_t M, int64_t N, int64_t K, float alpha, const qlinear_epilogue* epilogue, int path,
                          void* workspace, int64_t workspace_bytes, void* stream) {
  return nvfp4_gemm_impl(w_packed, w_scale, x, out, out_dtype, M, N, K, alpha, path, workspace, workspace_bytes,
                         stream, epilogue);
}

int qlinear_bf16_gemm_ws(const void* w, const void* x, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                         float alpha, const qlinear_epilogue* epilogue, int path, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  return bf16_gemm_impl(w, x, out, out_dtype, M, N, K, alpha, path, workspace, workspace_bytes, stream, epilogue);
}

}  // extern "C"
