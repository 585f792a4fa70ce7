"""Every output of the benchmarked full-size plans against the oracle.

The benchmark times the planner's plan with split K allowed
(GEMM_FLAG_SPLIT_K).  At bf16 4096^3 that is the 256 x 256 tile with
16-byte copies and 64 trips; at deep K it is the same tile with K cut into
ranges and the reduction kernel; FP8 4096^3 runs the 256 x 256 x 128 FP8
tile.  Here each of those plans computes the whole product once and every
one of its outputs is compared with the oracle's, which computes the whole
product on the host's cores (page "gizml:tile", the worked example at the
top of the page: every output of C is defined).

Two bars:
- Gaussian inputs (the workloads' own recipe): max floored relative error
  <= 1e-2 over every output;
- integer inputs in [-4, 4] through the same plan: every partial sum is an
  integer below 2^24, so the fp32 result is exact in any order and the
  output must equal the oracle's bit for bit.
"""
import numpy as np
import pytest
import torch

import gemm_workloads as gw
from gpu_helpers import as_bits, check_against_oracle, note, run

pytestmark = pytest.mark.gpu

FULL = ["bf16_4096_relu", "deepk_bf16_2048x16384", "fp8_4096_relu"]


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    return t


def integer_twin(w):
    """The workload's shape, types and epilogue with integer entries."""
    return gw.custom(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, gw.INT4,
                     seed=w.seed + 100, name=w.name + "_int")


@pytest.mark.parametrize("name", FULL)
def test_every_output_of_the_benchmarked_plan(tcg, name):
    w = gw.WORKLOADS[name]
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, flags=tcg.FLAG_SPLIT_K)
    note(f"{name}: comparing all {w.M * w.N} outputs with the oracle")
    worst = check_against_oracle(w, A, B, C)
    note(f"{name}: max floored relative error {worst:.3e} ({p.describe()})")


@pytest.mark.parametrize("name", FULL)
def test_benchmarked_plan_is_exact_on_integers(tcg, name):
    w = gw.WORKLOADS[name]
    wi = integer_twin(w)
    assert wi.exact
    A, B = gw.make_inputs(wi)
    C, _, p = run(tcg, A, B, wi, flags=tcg.FLAG_SPLIT_K)
    # the same plan as the Gaussian workload's (the plan depends only on
    # the shape, the types, the epilogue and the flags)
    p_ref = tcg.gemm_plan(tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                                        tcg.FLAG_SPLIT_K))
    assert p.describe() == p_ref.describe()
    check_against_oracle(wi, A, B, C)


def test_headline_plan_takes_the_16_byte_staged_path(tcg):
    """The headline plan stages its operands with 16-byte copies: the path
    the two tests above cover in full."""
    w = gw.WORKLOADS["bf16_4096_relu"]
    i = tcg.gemm_plan(tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                                    tcg.FLAG_SPLIT_K)).info()
    assert i.stages >= 2 and i.vec16 == 1
