"""The persistent short-K kernel (tile 11) on the GPU.

It runs the MFMA sequence of the 128 x 288 x 32 tile (tile 5): per output,
k-steps of 16 in ascending order over whole 32-deep trips, zero past K.  Its
results must therefore equal tile 5's bit for bit on every input, and tile
5 is itself pinned to the oracle and to the unstaged kernel by the other
parity tests.  The cases cover one to four blocks per workgroup (the
three-slot ring wraps after three), ragged M, N below 288, every K class
(2, 4 and 6 k-steps), relu and none, and the three output types; the
oracle checks the kernel directly on integer and Gaussian inputs, and a
guard band checks that rows past M and columns past N are never written.
"""
import numpy as np
import pytest
import torch

import gemm_workloads as gw
from gemm_workloads import BF16, EPI_NONE, EPI_RELU, F16, F32
from gpu_helpers import as_bits, check_against_oracle, check_sampled, note, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    return t


def blocks_per_workgroup(tcg, M):
    cus = tcg.gemm_device_caps_query(0).num_cus
    return -(-(-(-M // 128)) // cus)


# (M, N, K): M = 128 * CUs * b - r gives b blocks for most workgroups.
SHAPES = [(1, 288, 96), (127, 200, 40), (129, 96, 64), (5000, 136, 16), (32768, 288, 96),
          (65536 - 77, 192, 88), (98304 - 5, 288, 32), (129600, 288, 96), (131072 + 3, 8, 8)]
TYPES = [(F16, F16, EPI_NONE), (BF16, BF16, EPI_RELU), (F16, F32, EPI_RELU), (BF16, F32, EPI_NONE)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("in_dtype,out_dtype,epi", TYPES)
def test_same_bits_as_the_128x288x32_tile(tcg, M, N, K, in_dtype, out_dtype, epi):
    w = gw.custom(M, N, K, in_dtype, out_dtype, epi, gw.NORMAL, seed=M + 3 * N + 7 * K)
    A, B = gw.make_inputs(w)
    C11, _, p = run(tcg, A, B, w, tile=11)
    assert p.info().tile_id == 11
    note(f"blocks per workgroup: {blocks_per_workgroup(tcg, M)}")
    C5, _, _ = run(tcg, A, B, w, tile=5)
    assert np.array_equal(as_bits(C11), as_bits(C5))


@pytest.mark.parametrize("M,N,K", [(1000, 288, 96), (3000, 200, 40), (777, 96, 8)])
def test_exact_on_integers(tcg, M, N, K):
    w = gw.custom(M, N, K, F16, F32, EPI_RELU, gw.INT4, seed=M)
    A, B = gw.make_inputs(w)
    C, _, _ = run(tcg, A, B, w, tile=11)
    check_against_oracle(w, A, B, C)


@pytest.mark.parametrize("out_dtype", [F32, F16, BF16])
def test_gaussian_within_tolerance(tcg, out_dtype):
    w = gw.custom(3000, 288, 96, F16, out_dtype, EPI_NONE, gw.NORMAL, seed=31,
                  dist_b=gw.Dist("normal", 0.0, 96 ** -0.5))
    A, B = gw.make_inputs(w)
    C, _, _ = run(tcg, A, B, w, tile=11)
    check_against_oracle(w, A, B, C)


def test_many_blocks_sampled(tcg):
    """Four blocks per workgroup on most CUs, bf16 with relu, sampled."""
    w = gw.custom(129600, 264, 72, BF16, BF16, EPI_RELU, gw.NORMAL, seed=5)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w)
    assert p.info().tile_id == 11
    check_sampled(w, A, B, C)


@pytest.mark.parametrize("out_dtype", [F32, F16])
def test_guard_band_untouched(tcg, out_dtype):
    """Rows past M and columns past N are dropped by the buffer unit."""
    w = gw.custom(333, 200, 56, F16, out_dtype, EPI_RELU, gw.INT4, seed=7)
    A, B = gw.make_inputs(w)
    guard = 8192
    sentinel = 0x5A5A5A5A if out_dtype == F32 else 0x5A5A
    C, buf, _ = run(tcg, A, B, w, tile=11, guard=guard, sentinel=sentinel)
    raw = as_bits(buf)
    sent = np.array(sentinel, raw.dtype)
    assert np.all(raw[:guard] == sent) and np.all(raw[-guard:] == sent)
    check_against_oracle(w, A, B, C)


def test_misaligned_pointers_take_tile_5(tcg):
    """Operands not 16-byte aligned: the run takes tile 5's kernel with
    element copies, which gives the same bits."""
    w = gw.custom(2000, 288, 96, F16, F16, EPI_NONE, gw.NORMAL, seed=3)
    A, B = gw.make_inputs(w)
    C0, _, p = run(tcg, A, B, w, tile=11)
    C1, _, _ = run(tcg, A, B, w, plan=p, a_offset=1, b_offset=3)
    assert np.array_equal(as_bits(C0), as_bits(C1))
    check_against_oracle(w, A, B, C0)


def test_repeat_runs_identical(tcg):
    w = gw.custom(70000, 288, 96, F16, F16, EPI_NONE, gw.NORMAL, seed=8)
    A, B = gw.make_inputs(w)
    C0, _, p = run(tcg, A, B, w, tile=11)
    first = as_bits(C0)
    for _ in range(3):
        assert np.array_equal(as_bits(run(tcg, A, B, w, plan=p)[0]), first)


def test_misaligned_output_takes_tile_5(tcg):
    """C not 16-byte aligned (3 elements into its buffer): the run takes
    tile 5's kernel with element stores; same bits, guard band untouched."""
    w = gw.custom(3000, 200, 64, F16, F16, EPI_RELU, gw.NORMAL, seed=13)
    A, B = gw.make_inputs(w)
    C0, _, p = run(tcg, A, B, w, tile=11)
    C1, buf, _ = run(tcg, A, B, w, plan=p, guard=3, sentinel=0x5A5A)
    assert np.array_equal(as_bits(C0), as_bits(C1))
    raw = as_bits(buf)
    assert np.all(raw[:3] == np.int16(0x5A5A)) and np.all(raw[-3:] == np.int16(0x5A5A))


def test_autotune_counts_the_persistent_tile(tcg):
    """A short-K problem: the autotuner times tile 11 with the others and
    the plan it keeps computes the product."""
    tcg.gemm_tune_cache_clear()
    w = gw.custom(40000, 288, 96, F16, F16, EPI_NONE, gw.NORMAL, seed=14,
                  dist_b=gw.Dist("normal", 0.0, 96 ** -0.5))
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    C = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    desc = tcg.make_desc(w.M, w.N, w.K, F16, F16, EPI_NONE)
    assert tcg.gemm_plan_for_caps(tcg.make_desc(w.M, w.N, w.K, F16, F16, EPI_NONE, tile=11),
                                  tcg.gemm_device_caps_query(0)).info().tile_id == 11
    p = tcg.gemm_autotune(desc, Ad, Bd, C)
    note(f"autotune 40000x288x96 chose: {p.describe()}")
    C.fill_(float("nan"))
    tcg.gemm_run(p, Ad, Bd, C)
    torch.cuda.synchronize()
    check_against_oracle(w, A, B, C.cpu().reshape(1, w.M, w.N))
    tcg.gemm_tune_cache_clear()
