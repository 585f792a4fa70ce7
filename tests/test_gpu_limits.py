"""Parity at the limits of the kernels' 32-bit buffer offsets.

Every global access goes through a buffer resource whose size is clamped to
2^31 - 1 bytes, at byte offsets below 2^31 from a tile's (or band's) first
element; the planner refuses a tile whose rows would need larger offsets
(GEMM_E_SIZE).  These cases sit at those limits: an output and an operand
larger than 2 GiB (clamped resource sizes), and the largest K the 256 x 256
tile takes with 16-byte copies (row offsets just under 2^31).  Integer
inputs make every partial sum exact, so there is one correct result and the
comparisons with the oracle are bitwise.  Inputs are drawn on the GPU from
seeded generators and copied to the host for the oracle.
"""
import numpy as np
import pytest
import torch

import gemm_workloads as gw
import oracle
from gemm_workloads import BF16, EPI_NONE, EPI_RELU, F32
from gpu_helpers import check_sampled, note

pytestmark = pytest.mark.gpu

ONES = gw.Dist("randint", -1, 1)


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    return t


def _inputs(w, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    A = gw.draw((w.M, w.K), w.dist_a, w.in_dtype, g)
    B = gw.draw((w.K, w.N), w.dist_b, w.in_dtype, g)
    return A, B


def _run(tcg, w, A, B, flags=0, tile=0, split_k=0):
    p = tcg.gemm_plan(tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, flags,
                                    tile=tile, split_k=split_k))
    note(f"{w.name}: {p.describe()}")
    C = torch.full((w.M, w.N), float("nan"), dtype=gw.TORCH_DTYPE[w.out_dtype], device="cuda")
    wsb = p.info().workspace_bytes
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
    tcg.gemm_run_ex(p, A, B, C, workspace=ws)
    torch.cuda.synchronize()
    return C, p


def test_output_larger_than_2gib(tcg):
    # C: 24576^2 fp32 = 2.4 GB; the store resources of the first bands are clamped
    w = gw.custom(24576, 24576, 64, BF16, F32, EPI_RELU, gw.INT4, seed=71, name="c_over_2gib")
    A, B = _inputs(w, 71)
    C, _ = _run(tcg, w, A, B, tcg.FLAG_SPLIT_K)
    assert w.M * w.N * 4 > 2**31
    # every output: the sums are exact in fp32 (|sum| <= 64 * 16), so the
    # fp32 product on the GPU is the one correct result
    want = torch.relu(A.float() @ B.float())
    assert torch.equal(C, want)
    del want
    check_sampled(w, A.cpu(), B.cpu(), C.cpu().reshape(1, w.M, w.N), count=4096, seed=72)


def test_operand_larger_than_2gib(tcg):
    # A: 65792 x 16384 bf16 = 2.16 GB (the first row block's resource is
    # clamped); 257 row blocks of the 256 x 256 tile, planned as the
    # benchmark plans (split K allowed: a small last round)
    w = gw.custom(65792, 256, 16384, BF16, BF16, EPI_RELU, gw.INT4, seed=73, name="a_over_2gib")
    A, B = _inputs(w, 73)
    assert w.M * w.K * 2 > 2**31
    C, _ = _run(tcg, w, A, B, tcg.FLAG_SPLIT_K)
    check_sampled(w, A.cpu(), B.cpu(), C.cpu().reshape(1, w.M, w.N), count=4096, seed=74)
    # the last row block, every output
    want = oracle.gemm(A[-256:].cpu(), B.cpu(), 256, 256, w.K, BF16, BF16, EPI_RELU)[0]
    got = C[-256:].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_row_offsets_just_under_31_bits(tcg):
    # the 256 x 256 tile reads row r of its A block at byte offset r * K * 2:
    # with K = 4194296, the largest multiple of 8 it takes, row 255 starts
    # 2,139,090,960 bytes in, 0.4 % below 2^31 (K + 8 is refused with
    # GEMM_E_SIZE); entries in {-1, 0, 1} keep every partial sum exact
    # (|sum| <= K < 2^24)
    K = 4194296
    w = gw.custom(256, 64, K, BF16, BF16, EPI_NONE, ONES, seed=75, name="k_4194296")
    assert 255 * K * 2 + 8 * 16 < 2**31 and 256 * (K + 8) * 2 >= 2**31 - 1
    A, B = _inputs(w, 75)
    C, p = _run(tcg, w, A, B, tile=1, split_k=64)
    assert p.info().tile_id == 1 and p.info().vec16 == 1
    want = oracle.gemm(A.cpu(), B.cpu(), w.M, w.N, K, BF16, BF16, EPI_NONE)[0]
    got = C.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
