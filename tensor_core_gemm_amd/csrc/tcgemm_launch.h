// Host-visible declarations of the per-tile launchers (one translation unit
// per tile configuration instantiates the kernel template).
#pragma once

#include <hip/hip_runtime.h>

#include "tcgemm_kernel_args.h"

namespace tcg {

hipError_t launch_t1(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t2(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t3(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t4(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t5(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t6(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t7(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);

}  // namespace tcg
