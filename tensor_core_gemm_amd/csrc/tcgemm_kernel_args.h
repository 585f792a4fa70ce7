// Arguments of the GEMM kernels, shared by the host launcher and the device code.
#pragma once

#include <stdint.h>

namespace tcg {

// Kernel arguments (passed by value).
struct KArgs {
  const void* A;                         // [batch][M][K] operand elements (2 or 1 bytes)
  const void* B;                         // [batch][K][N]
  void* C;
  const float* bias;                     // N values added to every row before the activation, or null
  float* ws;                             // split-K partial sums [splits][batch][M][N], or null
  int64_t M, N, K;
  int64_t stride_a, stride_b, stride_c;  // elements between batch items
  int64_t tiles_m, tiles_n;
  int64_t batch;
  int64_t workgroups;                    // tiles_m * tiles_n * batch * splits
  int32_t trips;                         // ceil(K / BK): trips of the whole K range
  int32_t splits;                        // K ranges; 1: the kernel finishes C itself
  int32_t trips_per_split;               // trips of each K range (the last may have fewer)
  int32_t out_dtype;                     // 0 f32, 4 f16, 5 bf16
  int32_t act;                           // activation code (GEMM_EPI_*)
  int32_t group_m;                       // tile rows per group in the tile order
  int32_t xcd_remap;                     // 1: give each XCD a contiguous run of tiles
  int32_t vec_store4;                    // 1: stores of 4 consecutive elements of C are aligned
  int32_t vec_store16;                   // 1: 16-byte stores of whole chunks of C are aligned
  int32_t ws_vec;                        // 1: the same for the partial sums (N a multiple of 4)
};

// Arguments of the split-K reduction: C = act(sum over s of ws[s] + bias).
struct RArgs {
  const float* ws;
  void* C;
  const float* bias;
  int64_t M, N, batch, stride_c;
  int32_t splits;
  int32_t out_dtype;
  int32_t act;
  int32_t vec4;  // 1: N a multiple of 4 and C aligned for 4-element stores
};

}  // namespace tcg
