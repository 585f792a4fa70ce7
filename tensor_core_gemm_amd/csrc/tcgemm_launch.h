// Host-visible declarations of the per-tile launchers.  Two translation
// units per tile configuration instantiate the kernel template: launch_tN
// with the rounded epilogue (no bias; none or relu; split-K partial sums)
// and launch_tN_gen with the general one (bias, any activation).
#pragma once

#include <hip/hip_runtime.h>

#include "tcgemm_kernel_args.h"

namespace tcg {

hipError_t launch_t1(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t1_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t2(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t2_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t3(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t3_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t4(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t4_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t5(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t5_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t6(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t6_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t7(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t7_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t8(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t8_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t9(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t9_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t10(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t10_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);

hipError_t launch_t12(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t12_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t13(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);
hipError_t launch_t13_gen(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s);

// The persistent short-K kernel, tile 11 (tcgemm_shortk.hip): a.workgroups
// workgroups loop over a.tiles_m blocks of 128 rows.
hipError_t launch_t11(bool bf16, const KArgs& a, hipStream_t s);

// The split-K reduction (tcgemm_reduce.hip).
hipError_t launch_splitk_reduce(const RArgs& r, hipStream_t s);

}  // namespace tcg
