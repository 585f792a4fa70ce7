// Instantiates the GEMM kernels of tile configuration 13, general epilogue.
#include "tcgemm_kernel.h"
#include "tcgemm_launch.h"

namespace tcg {
hipError_t launch_t13_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s) {
  return launch_tile<13, true>(stages, vec16, bf16, a, s);
}
}  // namespace tcg
