"""Several host threads, each launching its own plans on its own stream at
once (a server's pattern).  Plans are immutable after creation and the
library's shared state (the device-capability cache, the tune cache) is
locked, so concurrent runs must give exactly the results of the same runs
made one at a time: every output is compared bit for bit with a
single-threaded run, which the other parity tests pin to the oracle.  Each
thread owns its inputs, outputs and split-K workspace (gemm_run_noalloc is
left out: its fixed array is shared by design).
"""
import threading

import numpy as np
import pytest
import torch

import gemm_workloads as gw
from gemm_workloads import BF16, EPI_GELU, EPI_NONE, EPI_RELU, F16, F32, FP8
from gpu_helpers import as_bits, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    return t


# (workload, flags name, tile, split, bias)
JOBS = [
    (gw.custom(2048, 2048, 1024, BF16, BF16, EPI_RELU, gw.NORMAL, seed=81), "none", 0, 0, False),
    (gw.custom(1000, 1000, 1000, F16, F32, EPI_RELU, gw.UNIT, seed=82), "none", 0, 0, False),
    (gw.custom(512, 520, 4096, BF16, F16, EPI_GELU, gw.NORMAL, seed=83), "none", 1, 4, True),
    (gw.custom(20000, 288, 96, F16, F16, EPI_NONE, gw.NORMAL, seed=84), "none", 0, 0, False),
    (gw.custom(1024, 1024, 2048, FP8, BF16, EPI_NONE, gw.NORMAL, seed=85), "split", 0, 0, False),
]
ITERS = 20


def _prepare(tcg, w, flags, tile, split, bias):
    A, B = gw.make_inputs(w)
    f = tcg.FLAG_SPLIT_K if flags == "split" else 0
    if bias:
        f |= tcg.FLAG_BIAS
    p = tcg.gemm_plan(tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, f,
                                    tile=tile, split_k=split))
    wsb = p.info().workspace_bytes
    b = gw.draw_bias(w.N, gw.NORMAL, seed=w.seed + 100).cuda() if bias else None
    return {"w": w, "p": p, "A": A.cuda(), "B": B.cuda(), "bias": b,
            "ws": torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda") if wsb else None,
            "C": torch.full((w.M, w.N), float("nan"), dtype=gw.TORCH_DTYPE[w.out_dtype], device="cuda")}


def _run(tcg, job, stream):
    tcg.gemm_run_ex(job["p"], job["A"], job["B"], job["C"], bias=job["bias"], workspace=job["ws"],
                    stream=stream)


def test_concurrent_streams_from_threads_match_single_threaded_runs(tcg):
    jobs = [_prepare(tcg, *j) for j in JOBS]
    for job in jobs:
        note(f"stream job {job['w'].name}: {job['p'].describe()}")
    # one at a time on the default stream
    want = []
    for job in jobs:
        _run(tcg, job, torch.cuda.current_stream())
        torch.cuda.synchronize()
        want.append(as_bits(job["C"].cpu()))
        job["C"].fill_(float("nan"))
    torch.cuda.synchronize()

    errors = []
    streams = [torch.cuda.Stream() for _ in jobs]
    start = threading.Barrier(len(jobs))

    def worker(i):
        try:
            job, s = jobs[i], streams[i]
            start.wait()
            for _ in range(ITERS):
                _run(tcg, job, s)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for job, ref in zip(jobs, want):
        assert np.array_equal(as_bits(job["C"].cpu()), ref), job["w"].name
