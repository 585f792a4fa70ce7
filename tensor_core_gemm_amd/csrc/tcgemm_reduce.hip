// Split-K reduction: C = act(ws[0] + ws[1] + ... + ws[splits-1] + bias),
// the partial sums added in ascending K-range order in fp32, then the same
// epilogue as the GEMM kernels.  Memory-bound: each lane reads `splits`
// runs of 16 bytes and writes 4 outputs (or 1 where N is not a multiple of 4).
#include <hip/hip_runtime.h>

#include "tcgemm_epilogue.h"
#include "tcgemm_kernel_args.h"
#include "tcgemm_launch.h"

namespace tcg {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kReduceThreads = 256;

__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(RArgs r) {
  const int64_t MN = r.M * r.N;
  const int64_t total = r.batch * MN;
  const int64_t split_stride = total;  // elements between consecutive K ranges
  const int64_t step = (int64_t)gridDim.x * kReduceThreads;
  const int osz = r.out_dtype == kOutF32 ? 4 : 2;
  if (r.vec4) {
    for (int64_t e = 4 * ((int64_t)blockIdx.x * kReduceThreads + threadIdx.x); e < total; e += 4 * step) {
      const int64_t b = e / MN, rem = e - b * MN;
      const int64_t n = rem % r.N;  // a multiple of 4; n + 3 < N
      f32x4 acc = *(const f32x4*)(r.ws + e);
      for (int s = 1; s < r.splits; ++s) {
        const f32x4 v = *(const f32x4*)(r.ws + s * split_stride + e);
        acc[0] += v[0];
        acc[1] += v[1];
        acc[2] += v[2];
        acc[3] += v[3];
      }
      float y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = epilogue_value(acc[q], r.bias, n + q, r.N, r.act);
      char* dst = (char*)r.C + (b * r.stride_c + rem) * osz;
      if (r.out_dtype == kOutF32) {
        *(f32x4*)dst = f32x4{y[0], y[1], y[2], y[3]};
      } else {
        const uint32_t lo = (uint32_t)to_out16(y[0], r.out_dtype) | ((uint32_t)to_out16(y[1], r.out_dtype) << 16);
        const uint32_t hi = (uint32_t)to_out16(y[2], r.out_dtype) | ((uint32_t)to_out16(y[3], r.out_dtype) << 16);
        *(u32x2*)dst = u32x2{lo, hi};
      }
    }
  } else {
    for (int64_t e = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x; e < total; e += step) {
      const int64_t b = e / MN, rem = e - b * MN;
      const int64_t n = rem % r.N;
      float acc = r.ws[e];
      for (int s = 1; s < r.splits; ++s) acc += r.ws[s * split_stride + e];
      const float y = epilogue_value(acc, r.bias, n, r.N, r.act);
      char* dst = (char*)r.C + (b * r.stride_c + rem) * osz;
      if (r.out_dtype == kOutF32)
        *(float*)dst = y;
      else
        *(uint16_t*)dst = to_out16(y, r.out_dtype);
    }
  }
}

}  // namespace

hipError_t launch_splitk_reduce(const RArgs& r, hipStream_t s) {
  const int64_t total = r.batch * r.M * r.N;
  const int64_t lanes = r.vec4 ? (total + 3) / 4 : total;
  int64_t blocks = (lanes + kReduceThreads - 1) / kReduceThreads;
  if (blocks > 65536) blocks = 65536;  // the loop strides over the rest
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((uint32_t)blocks), dim3(kReduceThreads), 0, s, r);
  return hipGetLastError();
}

}  // namespace tcg
