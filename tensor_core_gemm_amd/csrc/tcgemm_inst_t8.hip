// Instantiates the GEMM kernels of tile configuration 8 (FP8), rounded epilogue.
#include "tcgemm_kernel.h"
#include "tcgemm_launch.h"

namespace tcg {
hipError_t launch_t8(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s) {
  return launch_tile<8, false>(stages, vec16, bf16, a, s);
}
}  // namespace tcg
