"""Parity of the fused epilogues (bias row, activations) and of split K on
the GPU, through the C ABI, against the CPU oracle.

Activations and bias follow the page "gizml:tile" (Tile.add with
broadcasting, Tile.relu, Tile.gelu, Tile.geluErf, Tile.sigmoid, Tile.tanh).
Split K reassociates the fold over k (ranges summed in ascending order), so
it is checked bit for bit where the arithmetic is exact (integer operands),
within the tolerance elsewhere, and every path of one split plan must give
the same bits (staging copies values unchanged).
"""
import math

import numpy as np
import pytest
import torch

import gemm_workloads as gw
import oracle
from gemm_workloads import (BF16, EPI_GELU, EPI_GELU_ERF, EPI_NONE, EPI_RELU, EPI_SIGMOID,
                            EPI_TANH, F16, F32)
from gpu_helpers import as_bits, as_values, check_against_oracle, check_sampled, note, run

pytestmark = pytest.mark.gpu

ACTS = [EPI_NONE, EPI_RELU, EPI_GELU, EPI_GELU_ERF, EPI_SIGMOID, EPI_TANH]


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    return t


def unit_sum(K):
    """Operands whose products sum to about N(0, 1): the activations' whole range."""
    return gw.Dist("normal", 0.0, K ** -0.25)


@pytest.mark.parametrize("out_dtype", [F32, F16, BF16])
@pytest.mark.parametrize("epi", ACTS)
def test_bias_and_activation_match_the_oracle(tcg, epi, out_dtype):
    K = 130
    w = gw.custom(300, 260, K, BF16, out_dtype, epi, unit_sum(K), seed=40 + epi)
    A, B = gw.make_inputs(w)
    bias = gw.draw_bias(w.N, gw.NORMAL, seed=epi)
    C, _, p = run(tcg, A, B, w, bias=bias)
    check_against_oracle(w, A, B, C, bias=bias)
    Cu, _, _ = run(tcg, A, B, w, bias=bias, flags=tcg.FLAG_UNSTAGED, tile=p.info().tile_id)
    assert np.array_equal(as_bits(C), as_bits(Cu))


def _condition(epi, x):
    """|x f'(x) / f(x)|, the relative condition number of the activation, in
    float64 by central differences (a tolerance scale, not a reference)."""
    from scipy import special
    f = {EPI_GELU: lambda t: 0.5 * t * (1 + np.tanh(np.sqrt(2 / np.pi) * (t + 0.044715 * t ** 3))),
         EPI_GELU_ERF: lambda t: 0.5 * t * special.erfc(-t / np.sqrt(2)),
         EPI_SIGMOID: special.expit, EPI_TANH: np.tanh}[epi]
    x = x.astype(np.float64)
    h = 1e-6 * np.maximum(1.0, np.abs(x))
    d = (f(x + h) - f(x - h)) / (2 * h)
    fx = f(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        k = np.abs(x * d / fx)
    return np.where(np.isfinite(k), k, 0.0)


@pytest.mark.parametrize("epi", [EPI_GELU, EPI_GELU_ERF, EPI_SIGMOID, EPI_TANH])
def test_activations_within_a_few_ulp_on_exact_inputs(tcg, epi):
    """A = I, so each output's fp32 input to the activation is an exact fp16
    value of the grid k / 256 in [-8, 8): the device's fp32 activation is
    compared with the oracle's.  The page puts their error at two to three ulp;
    an fp32 evaluation cannot do better than the rounding of its inner
    argument amplified by the function's condition number k(x) (large in the
    GELU forms' negative tail, where the result decays like e^-(2u)), so the
    bar is 4 ulp plus 2 k(x) ulp.  Where the oracle's literal GELU formulas
    cancel in double precision (1 + tanh, 1 + erf far in the tail) it is
    accurate to about 1e-16 absolute, so a difference below 1e-15 passes."""
    M = K = 64
    N = 64
    grid = (np.arange(M * N, dtype=np.float32) - 2048.0) / 256.0
    A = torch.eye(M, dtype=torch.float16)
    B = torch.from_numpy(grid.reshape(K, N)).to(torch.float16)
    w = gw.custom(M, N, K, F16, F32, epi, gw.NORMAL, name=f"grid_{epi}")
    C, _, _ = run(tcg, A, B, w)
    want = oracle.gemm(A, B, M, N, K, F16, F32, epi).reshape(M, N)
    got = as_values(C).reshape(M, N)
    ia = got.view(np.int32).astype(np.int64)
    ib = want.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7fffffff), ia)
    ib = np.where(ib < 0, -(ib & 0x7fffffff), ib)
    ulps = np.abs(ia - ib)
    x = grid.reshape(K, N)
    allowed = 4 + 2 * _condition(epi, x)
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bad = (ulps > allowed) & (diff > 1e-15)
    assert not bad.any(), (int(bad.sum()), x[bad][:5], ulps[bad][:5], allowed[bad][:5])
    note(f"max ulps {ulps.max()}, where k(x) <= 1: {ulps[_condition(epi, x) <= 1].max()}")


def test_bias_on_exact_integer_sums(tcg):
    w = gw.custom(257, 300, 200, F16, F32, EPI_RELU, gw.INT4, seed=61)
    A, B = gw.make_inputs(w)
    bias = gw.draw_bias(w.N, gw.Dist("randint", -20, 20), seed=3)
    C, _, _ = run(tcg, A, B, w, bias=bias)
    check_against_oracle(w, A, B, C, bias=bias)  # exact: integer sums and bias


def test_bias_is_shared_by_batch_items(tcg):
    w = gw.custom(130, 70, 90, BF16, F32, EPI_TANH, unit_sum(90), seed=62, batch=3)
    A, B = gw.make_inputs(w)
    bias = gw.draw_bias(w.N, gw.NORMAL, seed=4)
    C, _, _ = run(tcg, A, B, w, bias=bias)
    check_against_oracle(w, A, B, C, bias=bias)


@pytest.mark.parametrize("tile,split", [(1, 2), (1, 5), (2, 3), (3, 8), (3, 2)])
def test_split_k_is_exact_on_integers(tcg, tile, split):
    w = gw.custom(300, 288, 2048, F16, F32, EPI_RELU, gw.INT4, seed=70 + split)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, tile=tile, split_k=split)
    assert p.info().split_k == split and p.info().workspace_bytes == split * 300 * 288 * 4
    check_against_oracle(w, A, B, C)  # exact


@pytest.mark.parametrize("out_dtype", [F32, BF16])
def test_split_k_float_within_tolerance_and_paths_agree(tcg, out_dtype):
    w = gw.custom(300, 260, 4000, BF16, out_dtype, EPI_RELU, gw.NORMAL, seed=71)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, tile=2, split_k=4)
    assert p.info().split_k == 4
    check_against_oracle(w, A, B, C)
    for flags in (tcg.FLAG_UNSTAGED, tcg.FLAG_FORCE_STAGES_1):
        C2, _, _ = run(tcg, A, B, w, tile=2, split_k=4, flags=flags)
        assert np.array_equal(as_bits(C), as_bits(C2)), flags
    # the workspace's contents on entry do not matter
    C3, _, _ = run(tcg, A, B, w, tile=2, split_k=4, ws_fill=1e30)
    assert np.array_equal(as_bits(C), as_bits(C3))


def test_split_k_with_bias_activation_batch_and_ragged_n(tcg):
    # N = 77: not a multiple of 4, so the reduction takes its one-element path
    w = gw.custom(150, 77, 1000, F16, F16, EPI_GELU, unit_sum(1000), seed=72, batch=2)
    A, B = gw.make_inputs(w)
    bias = gw.draw_bias(w.N, gw.NORMAL, seed=5)
    C, _, p = run(tcg, A, B, w, tile=3, split_k=3, bias=bias)
    assert p.info().split_k == 3
    check_against_oracle(w, A, B, C, bias=bias)
    Cu, _, _ = run(tcg, A, B, w, tile=3, split_k=3, bias=bias, flags=tcg.FLAG_UNSTAGED)
    assert np.array_equal(as_bits(C), as_bits(Cu))


def test_split_k_tanh_output_where_the_sum_cancels(tcg):
    # a random split problem whose output (268, 88) cancels to about 0.0103
    # against s = 44: the tolerance's floor carried through tanh's slope
    # admits the oracle's own fold error there (test_tolerance.py)
    w = gw.custom(516, 165, 1958, F16, F16, EPI_TANH, gw.NORMAL, seed=5471)
    A, B = gw.make_inputs(w)
    bias = gw.draw_bias(w.N, gw.NORMAL, seed=6471)
    C, _, p = run(tcg, A, B, w, tile=3, split_k=8, bias=bias)
    assert p.info().split_k == 8
    check_against_oracle(w, A, B, C, bias=bias)


def test_split_k_larger_than_the_trips_is_capped(tcg):
    w = gw.custom(70, 90, 100, F16, F32, EPI_NONE, gw.INT4, seed=73)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, tile=3, split_k=8)
    assert p.info().trips == 2 and p.info().split_k == 2
    check_against_oracle(w, A, B, C)


def test_deep_k_full_size_with_the_planners_split(tcg):
    w = gw.WORKLOADS["deepk_bf16_2048x16384"]
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, tile=1, split_k=4)
    assert p.info().split_k == 4 and p.info().workgroups == 256
    check_sampled(w, A, B, C)
    C2, _, _ = run(tcg, A, B, w, plan=p)
    assert np.array_equal(as_bits(C), as_bits(C2))


def test_run_ex_errors(tcg):
    dev = torch.device("cuda")
    A = torch.zeros(64 * 512, dtype=torch.float16, device=dev)
    B = torch.zeros(512 * 64, dtype=torch.float16, device=dev)
    C = torch.zeros(64 * 64, dtype=torch.float32, device=dev)
    bias = torch.zeros(64, dtype=torch.float32, device=dev)
    pb = tcg.gemm_plan(tcg.make_desc(64, 64, 512, F16, F32, EPI_RELU, tcg.FLAG_BIAS))
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_run(pb, A, B, C)  # the plan needs a bias
    assert e.value.code == tcg.GEMM_E_ARG
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_run_ex(pb, A, B, C, bias=C[:64])  # bias inside C
    assert e.value.code == tcg.GEMM_E_ALIAS
    tcg.gemm_run_ex(pb, A, B, C, bias=bias)
    ps = tcg.gemm_plan(tcg.make_desc(64, 64, 512, F16, F32, EPI_NONE, 0, tile=3, split_k=4))
    need = ps.info().workspace_bytes
    assert need == 4 * 64 * 64 * 4
    ws = torch.zeros(need // 4 + 128, dtype=torch.float32, device=dev)
    for kw in (dict(), dict(workspace=ws, workspace_bytes=need - 4),
               dict(workspace=ws.data_ptr() + 4, workspace_bytes=need)):
        with pytest.raises(tcg.GemmError) as e:
            tcg.gemm_run_ex(ps, A, B, C, **kw)
        assert e.value.code == tcg.GEMM_E_WORKSPACE, kw
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_run(ps, A, B, C)
    assert e.value.code == tcg.GEMM_E_WORKSPACE
    big = torch.zeros(need // 4 + 64 * 64, dtype=torch.float32, device=dev)
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_run_ex(ps, A, B, big[:4096], workspace=big, workspace_bytes=need)  # C in it
    assert e.value.code == tcg.GEMM_E_ALIAS
    tcg.gemm_run_ex(ps, A, B, C, workspace=ws)
    torch.cuda.synchronize()


def test_matmul_binding_with_bias_activation_and_split(tcg):
    w = gw.custom(200, 136, 512, BF16, F32, EPI_SIGMOID, unit_sum(512), seed=80)
    A, B = gw.make_inputs(w)
    bias = gw.draw_bias(w.N, gw.NORMAL, seed=6)
    note("matmul sigmoid + bias + split 2")
    C = tcg.matmul(A.cuda(), B.cuda(), act="sigmoid", bias=bias.cuda(), out_dtype=torch.float32,
                   split_k=2)
    torch.cuda.synchronize()
    check_against_oracle(w, A, B, C.cpu().reshape(1, w.M, w.N), bias=bias)
