// Arguments of the GEMM kernel, shared by the host launcher and the device code.
#pragma once

#include <stdint.h>

namespace tcg {

// Kernel arguments (passed by value).
struct KArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int64_t M, N, K;
  int64_t stride_a, stride_b, stride_c;  // elements between batch items
  int64_t tiles_m, tiles_n;
  int64_t workgroups;                    // tiles_m * tiles_n * batch
  int32_t trips;                         // ceil(K / BK)
  int32_t out_dtype;                     // 0 f32, 4 f16, 5 bf16
  int32_t relu;
  int32_t group_m;                       // tile rows per group in the tile order
  int32_t xcd_remap;                     // 1: give each XCD a contiguous run of tiles
  int32_t vec_store4;                    // 1: stores of 4 consecutive elements are aligned
  int32_t vec_store16;                   // 1: 16-byte stores of whole chunks are aligned
};

}  // namespace tcg
