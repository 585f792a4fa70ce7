"""gemm_run under HIP graph capture.

gemm_run allocates nothing, issues no memset and launches only kernels on
the caller's stream (a split plan also launches its reduction), so a HIP
graph can capture it.  The graph is replayed several times with eager work
and synchronisations between the replays, and every replay must give the
eager result bit for bit.
"""
import numpy as np
import pytest
import torch

import gemm_workloads as gw
from gemm_workloads import BF16, EPI_NONE, EPI_RELU, F16
from gpu_helpers import as_bits, check_against_oracle, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    return t


CASES = [
    # (workload, planner may split, tile, split): a single-kernel plan, a
    # split plan (GEMM plus reduction), the persistent short-K tile, and the
    # planner's split tail (the unsplit rows, then the last round's rows
    # split in K, then their reduction: three launches)
    (gw.custom(1000, 1000, 1000, F16, F16, EPI_RELU, gw.NORMAL, seed=41), False, 0, 0),
    (gw.custom(512, 512, 8192, BF16, BF16, EPI_NONE, gw.NORMAL, seed=42), False, 0, 4),
    (gw.custom(40000, 288, 96, F16, F16, EPI_NONE, gw.NORMAL, seed=43), False, 11, 0),
    (gw.custom(4352, 4352, 2048, BF16, BF16, EPI_RELU, gw.NORMAL, seed=44), True, 0, 0),
]


@pytest.mark.parametrize("w,may_split,tile,split", CASES, ids=["single", "split", "short_k", "split_tail"])
def test_captured_runs_replay_the_eager_result(tcg, w, may_split, tile, split):
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    odt = gw.TORCH_DTYPE[w.out_dtype]
    flags = tcg.FLAG_SPLIT_K if may_split else 0
    p = tcg.gemm_plan(tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, flags,
                                    tile=tile, split_k=split))
    note(f"graph capture {w.name}: {p.describe()}")
    if may_split:
        assert p.info().tail_rows > 0  # the case is the split tail
    ws_bytes = p.info().workspace_bytes
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()

    def launch(C):
        if ws_bytes:
            tcg.gemm_run_ex(p, Ad, Bd, C, workspace=ws, stream=s)
        else:
            tcg.gemm_run(p, Ad, Bd, C, s)

    C_eager = torch.empty((w.M, w.N), dtype=odt, device="cuda")
    with torch.cuda.stream(s):
        launch(C_eager)
    torch.cuda.synchronize()
    eager = as_bits(C_eager.cpu())
    check_against_oracle(w, A, B, C_eager.cpu().reshape(1, w.M, w.N))

    C = torch.empty((w.M, w.N), dtype=odt, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        launch(C)
    for r in range(4):
        C.fill_(float("nan"))           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(as_bits(C.cpu()), eager), f"replay {r}"
