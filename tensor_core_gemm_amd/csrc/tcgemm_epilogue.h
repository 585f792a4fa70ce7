// The epilogue applied to each fp32 sum: bias, activation, rounding to the
// output storage type.  Shared by the GEMM kernels and the split-K
// reduction so that every path rounds the same values the same way.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tcg {

constexpr int kOutF32 = 0, kOutF16 = 4, kOutBF16 = 5;
// Activation codes (the ABI's GEMM_EPI_* values).
constexpr int kActNone = 0, kActRelu = 1, kActGelu = 2, kActGeluErf = 3, kActSigmoid = 4, kActTanh = 5;

// Element-wise activations of the page "gizml:tile" (Tile.relu, Tile.gelu,
// Tile.geluErf, Tile.sigmoid, Tile.tanh), in fp32 with the device library's
// expf / tanhf / erfcf.  Each is written in a form without cancellation:
//   gelu (tanh form)  x (1 + tanh u) / 2 = x / (1 + e^(-2u)),
//                     u = sqrt(2/pi) (x + 0.044715 x^3)
//   gelu (erf form)   x (1 + erf(x / sqrt 2)) / 2 = x erfc(-x / sqrt 2) / 2
//   sigmoid           1 / (1 + e^(-x))
// relu maps NaN and -0 to +0 (max with a NaN gives the other operand).
__device__ __forceinline__ float activate(float v, int act) {
  switch (act) {
    case kActRelu:
      return v > 0.0f ? v : 0.0f;
    case kActGelu: {
      const float u = 0.7978845608028654f * (v + 0.044715f * (v * v * v));
      return v / (1.0f + expf(-2.0f * u));
    }
    case kActGeluErf:
      return 0.5f * v * erfcf(-0.7071067811865476f * v);
    case kActSigmoid:
      return 1.0f / (1.0f + expf(-v));
    case kActTanh:
      return tanhf(v);
    default:
      return v;
  }
}

// y = act(v + bias[n]) (no addition without a bias, so -0 stays -0).
__device__ __forceinline__ float epilogue_value(float v, const float* bias, int64_t n, int64_t N, int act) {
  if (bias) v += n < N ? bias[n] : 0.0f;
  return activate(v, act);
}

// The same for the four consecutive columns n .. n+3 of one row; one branch
// on the activation for all four (smaller code where it is inlined often).
__device__ __forceinline__ void epilogue4(float (&y)[4], const float* bias, int64_t n, int64_t N, int act) {
  if (bias) {
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] += n + q < N ? bias[n + q] : 0.0f;
  }
  switch (act) {
    case kActNone:
      break;
    case kActRelu:
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = activate(y[q], kActRelu);
      break;
    case kActGelu:
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = activate(y[q], kActGelu);
      break;
    case kActGeluErf:
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = activate(y[q], kActGeluErf);
      break;
    case kActSigmoid:
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = activate(y[q], kActSigmoid);
      break;
    default:
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = activate(y[q], kActTanh);
      break;
  }
}

__device__ __forceinline__ uint16_t to_out16(float v, int out_dtype) {
  return out_dtype == kOutBF16 ? __builtin_bit_cast(uint16_t, (__bf16)v)
                               : __builtin_bit_cast(uint16_t, (_Float16)v);
}

}  // namespace tcg
