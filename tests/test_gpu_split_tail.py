"""Plans whose last rows run as a second launch with K split.

4608^3 on the 256 x 256 tile makes 324 output tiles: one whole round on
256 CUs and a last round of 68.  With GEMM_FLAG_SPLIT_K the planner runs the
first 3584 rows (14 whole tile rows) unsplit and the last 1024 rows in three
K ranges, so that the last round occupies more CUs.  The rows above the tail
must give the unsplit plan's bits and the tail rows the bits of a plan split
in three; sampled outputs of both parts match the oracle (exactly on
integer inputs).  Both launches and the reduction run on the caller's
stream, so the plan also replays from a captured graph.
"""
import numpy as np
import pytest
import torch

import gemm_workloads as gw
from gemm_workloads import BF16, EPI_GELU, EPI_RELU, F16, F32
from gpu_helpers import as_bits, check_sampled, note, run

pytestmark = pytest.mark.gpu

M = N = K = 4608
HEAD = 3584


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    if t.gemm_device_caps_query(0).num_cus != 256:
        pytest.skip("the tail split of 4608^3 is planned for 256 CUs")
    return t


def tail_desc(tcg, w, flags=0):
    return tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, flags | tcg.FLAG_SPLIT_K)


def test_the_plan_splits_the_last_round(tcg):
    w = gw.custom(M, N, K, BF16, BF16, EPI_RELU, gw.NORMAL)
    i = tcg.gemm_plan(tail_desc(tcg, w)).info()
    assert (i.tile_id, i.split_k, i.tail_rows, i.tail_split) == (1, 1, M - HEAD, 3)
    assert i.tiles_m * 256 == HEAD


@pytest.mark.parametrize("in_dtype,out_dtype", [(BF16, BF16), (F16, F32)])
def test_head_and_tail_bits(tcg, in_dtype, out_dtype):
    w = gw.custom(M, N, K, in_dtype, out_dtype, EPI_RELU, gw.NORMAL, seed=71)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, flags=tcg.FLAG_SPLIT_K)
    assert p.info().tail_rows == M - HEAD
    check_sampled(w, A, B, C)
    C1, _, _ = run(tcg, A, B, w, tile=1, split_k=1)
    assert np.array_equal(as_bits(C[:, :HEAD]), as_bits(C1[:, :HEAD]))
    C3, _, p3 = run(tcg, A, B, w, tile=1, split_k=3)
    assert p3.info().split_k == 3
    assert np.array_equal(as_bits(C[:, HEAD:]), as_bits(C3[:, HEAD:]))


def test_exact_on_integers(tcg):
    # sums of at most 16 * 4608 in magnitude: exact in fp32 in any order
    w = gw.custom(M, N, K, F16, F32, EPI_RELU, gw.INT4, seed=72)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, flags=tcg.FLAG_SPLIT_K)
    assert p.info().tail_rows == M - HEAD
    check_sampled(w, A, B, C, count=8192)
    # every row of the tail's first and last tile rows, against the oracle
    bi = np.zeros(2 * N, np.int64)
    ii = np.concatenate([np.full(N, HEAD), np.full(N, M - 1)])
    jj = np.concatenate([np.arange(N), np.arange(N)])
    import oracle
    want, _ = oracle.gemm_sampled(A, B, M, N, K, w.in_dtype, w.out_dtype, w.epilogue, bi, ii, jj)
    assert np.array_equal(C.numpy()[bi, ii, jj], oracle.to_float(w.out_dtype, want))


def test_bias_and_gelu_in_both_parts(tcg):
    w = gw.custom(M, N, K, BF16, BF16, EPI_GELU, gw.NORMAL, seed=73)
    A, B = gw.make_inputs(w)
    bias = torch.from_numpy(np.random.default_rng(73).standard_normal(N).astype(np.float32))
    C, _, p = run(tcg, A, B, w, flags=tcg.FLAG_SPLIT_K, bias=bias)
    assert p.info().tail_rows == M - HEAD
    check_sampled(w, A, B, C, bias=bias)


def test_the_workspace_is_checked(tcg):
    w = gw.custom(M, N, K, BF16, BF16, EPI_RELU, gw.NORMAL)
    p = tcg.gemm_plan(tail_desc(tcg, w))
    need = p.info().workspace_bytes
    assert need == 3 * (M - HEAD) * N * 4
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((K, N), dtype=torch.bfloat16, device="cuda")
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_run_ex(p, A, B, C, workspace=small)
    assert e.value.code == tcg.GEMM_E_WORKSPACE
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_run(p, A, B, C)
    assert e.value.code == tcg.GEMM_E_WORKSPACE


def test_captured_runs_replay_the_eager_result(tcg):
    w = gw.custom(M, N, K, BF16, BF16, EPI_RELU, gw.NORMAL, seed=74)
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    p = tcg.gemm_plan(tail_desc(tcg, w))
    note(f"graph capture {w.name}: {p.describe()}")
    ws = torch.empty(p.info().workspace_bytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    C_eager = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):
        tcg.gemm_run_ex(p, Ad, Bd, C_eager, workspace=ws, stream=s)
    torch.cuda.synchronize()
    eager = as_bits(C_eager.cpu())
    C = torch.empty_like(C_eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tcg.gemm_run_ex(p, Ad, Bd, C, workspace=ws, stream=s)
    for r in range(3):
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(as_bits(C.cpu()), eager), f"replay {r}"


def test_fp8_tail_exact_on_integers(tcg):
    # FP8 operands on the 256 x 256 x 128 tile: 4608 x 4608 x 8192 runs its
    # last 1024 rows in 3 K ranges; sums of at most 16 * 8192 are exact
    w = gw.custom(4608, 4608, 8192, gw.FP8, F32, EPI_RELU, gw.INT4, seed=75)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, flags=tcg.FLAG_SPLIT_K)
    i = p.info()
    assert (i.tile_id, i.tail_rows, i.tail_split) == (8, 1024, 3)
    check_sampled(w, A, B, C, count=8192)
    C1, _, _ = run(tcg, A, B, w, tile=8, split_k=1)
    assert np.array_equal(as_bits(C), as_bits(C1))
