// The fused-epilogue descriptor shared by the C ABI and the kernels (a plain
// struct passed to kernels by value).
#pragma once

#include <stdint.h>

namespace qlinear {

// Element-wise work fused into the output store of a GEMM, applied to the
// float32 value of output element (m, n) before its single rounding:
//   v = alpha * acc;  v *= row_scale[m];  v *= col_scale[n];  v += bias[n];
//   v = act(v);  v += residual[m * ld + n]
// Every pointer may be null (step skipped).  act: 0 none, 1 ReLU, 2 SiLU
// (v / (1 + e^-v)), 3 GELU, tanh form.  `on` is nonzero when any step is
// present; kernels test it once, uniformly.
struct Epilogue {
  const float* row_scale = nullptr;
  const float* col_scale = nullptr;
  const uint16_t* bias = nullptr;  // bfloat16 [N]
  const void* residual = nullptr;  // float32 or bfloat16 (res_bf16) [M, ld]
  int64_t ld = 0;
  int act = 0;
  int res_bf16 = 0;
  int on = 0;
};

}  // namespace qlinear
