"""gemm_run_noalloc: the entry point for callers that cannot allocate device
memory.  It runs the same plan as gemm_run_ex, with the split-K workspace
taken from the library's fixed device array, so its output must equal
gemm_run_ex's bit for bit (and both are pinned to the oracle by the other
parity tests).  Two calls in a row, the second on a smaller problem, check
that the array's left-over contents from one call do not reach the next.
"""
import numpy as np
import pytest
import torch

import gemm_workloads as gw
from gemm_workloads import BF16, EPI_GELU, EPI_NONE, EPI_RELU, F16, F32
from gpu_helpers import as_bits, check_against_oracle, note

import tensor_core_gemm_amd as tcg


def _run_both(w, tile, split, bias=None, flags=0):
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    if bias is not None:
        flags |= tcg.FLAG_BIAS
    p = tcg.gemm_plan(tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, flags,
                                    tile=tile, split_k=split))
    info = p.info()
    note(f"noalloc {w.name}: {p.describe()}")
    assert info.workspace_bytes <= tcg.NOALLOC_SCRATCH_BYTES
    odt = gw.TORCH_DTYPE[w.out_dtype]
    bias_d = bias.cuda() if bias is not None else None
    C_ex = torch.full((w.M, w.N), float("nan"), dtype=odt, device="cuda")
    ws = (torch.full((max(info.workspace_bytes, 4) // 4,), float("nan"), device="cuda")
          if info.workspace_bytes else None)
    tcg.gemm_run_ex(p, Ad, Bd, C_ex, bias=bias_d, workspace=ws)
    C_na = torch.full((w.M, w.N), float("nan"), dtype=odt, device="cuda")
    tcg.gemm_run_noalloc(p, Ad, Bd, C_na, bias=bias_d)
    torch.cuda.synchronize()
    return A, B, C_ex.cpu(), C_na.cpu(), info


@pytest.mark.gpu
def test_noalloc_equals_gemm_run_ex_on_two_calls_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tcg.check_runtime()
    cases = [
        (gw.custom(600, 520, 4096, BF16, BF16, EPI_RELU, gw.NORMAL, seed=71, name="na_big"), 1, 4),
        (gw.custom(200, 136, 1024, F16, F32, EPI_NONE, gw.NORMAL, seed=72, name="na_small"), 3, 2),
    ]
    for w, tile, split in cases:
        A, B, C_ex, C_na, info = _run_both(w, tile, split)
        assert info.split_k == split and info.workspace_bytes > 0
        assert np.array_equal(as_bits(C_na), as_bits(C_ex)), w.name
        check_against_oracle(w, A, B, C_na.reshape(1, w.M, w.N))


@pytest.mark.gpu
def test_noalloc_full_size_split_plan_and_epilogues():
    """The deep-K workload's benchmarked split plan (the largest workspace
    the array is sized for), a split with bias and gelu, and a plan with no
    split (no scratch at all)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = gw.WORKLOADS["deepk_bf16_2048x16384"]
    plan = tcg.gemm_plan(tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                                       tcg.FLAG_SPLIT_K))
    i = plan.info()
    A, B, C_ex, C_na, _ = _run_both(w, i.tile_id, i.split_k)
    assert np.array_equal(as_bits(C_na), as_bits(C_ex))
    wg = gw.custom(300, 264, 2048, BF16, BF16, EPI_GELU, gw.NORMAL, seed=73, name="na_gelu")
    bias = gw.draw_bias(wg.N, gw.NORMAL, 74)
    _, _, C_ex, C_na, info = _run_both(wg, 1, 3, bias=bias)
    assert info.split_k == 3
    assert np.array_equal(as_bits(C_na), as_bits(C_ex))
    wn = gw.custom(256, 256, 256, F16, F32, EPI_RELU, gw.INT4, seed=75, name="na_nosplit")
    A, B, C_ex, C_na, info = _run_both(wn, 0, 0)
    assert info.workspace_bytes == 0
    assert np.array_equal(as_bits(C_na), as_bits(C_ex))
    check_against_oracle(wn, A, B, C_na.reshape(1, wn.M, wn.N))


@pytest.mark.gpu
def test_noalloc_under_graph_capture_replays_the_eager_result():
    """The callers this entry point is for include code under HIP graph
    capture.  A split-tail plan (three launches, the partial sums in the
    fixed array) is called once eagerly, then captured; between replays an
    eager call of another split plan overwrites the array, and every replay
    must still give the eager result bit for bit."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = gw.custom(4352, 4352, 2048, BF16, BF16, EPI_RELU, gw.NORMAL, seed=76, name="na_graph")
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    p = tcg.gemm_plan(tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                                    tcg.FLAG_SPLIT_K))
    info = p.info()
    note(f"noalloc graph {w.name}: {p.describe()}")
    assert info.tail_rows > 0 and 0 < info.workspace_bytes <= tcg.NOALLOC_SCRATCH_BYTES
    wo = gw.custom(512, 1024, 4096, BF16, BF16, EPI_NONE, gw.NORMAL, seed=77, name="na_other")
    Ao, Bo = (t.cuda() for t in gw.make_inputs(wo))
    po = tcg.gemm_plan(tcg.make_desc(wo.M, wo.N, wo.K, wo.in_dtype, wo.out_dtype, wo.epilogue, 0,
                                     tile=1, split_k=4))
    Co = torch.empty((wo.M, wo.N), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()

    C_eager = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):
        tcg.gemm_run_noalloc(p, Ad, Bd, C_eager, stream=s)
    torch.cuda.synchronize()
    eager = as_bits(C_eager.cpu())
    check_against_oracle(w, A, B, C_eager.cpu().reshape(1, w.M, w.N))

    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tcg.gemm_run_noalloc(p, Ad, Bd, C, stream=s)
    for r in range(4):
        C.fill_(float("nan"))
        tcg.gemm_run_noalloc(po, Ao, Bo, Co)    # eager work that overwrites the array
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(as_bits(C.cpu()), eager), f"replay {r}"


def test_noalloc_refuses_a_workspace_beyond_the_array():
    """A plan whose partial sums exceed the fixed array is refused with
    GEMM_E_SCRATCH before any device call (so this runs without a GPU)."""
    caps = tcg.make_caps()
    p = tcg.gemm_plan_for_caps(tcg.make_desc(4096, 4096, 16384, BF16, BF16, EPI_NONE, 0,
                                             tile=1, split_k=4), caps)
    assert p.info().workspace_bytes > tcg.NOALLOC_SCRATCH_BYTES
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_run_noalloc(p, 1 << 20, 2 << 20, 3 << 20, stream=0)
    assert e.value.code == tcg.GEMM_E_SCRATCH
