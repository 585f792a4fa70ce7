"""The autotuner on the GPU (page "gizml:tile", tune: each configuration
timed on this GPU for these shapes, the fastest kept and cached; every
configuration must compute the same result)."""
import numpy as np
import pytest
import torch

import gemm_workloads as gw
import oracle
from gemm_workloads import BF16, EPI_NONE, EPI_RELU, F16, F32
from gpu_helpers import as_bits, check_against_oracle, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    return t


def test_every_candidate_gives_the_same_bits_on_integers(tcg):
    """Integer operands with sums below 2^24: every tile and every split
    computes the one exact result."""
    M, N, K = 300, 200, 1024
    w = gw.custom(M, N, K, F16, F32, EPI_RELU, gw.INT4, seed=90)
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    want = oracle.gemm(A, B, M, N, K, F16, F32, EPI_RELU).reshape(M, N)
    for tile in (1, 2, 3, 4, 5, 6, 7, 12, 13):  # the 16-bit tiles (8-10 take FP8 operands; 11 short K)
        for split in (1, 2, 4, 8, 16):
            p = tcg.gemm_plan(tcg.make_desc(M, N, K, F16, F32, EPI_RELU, 0, tile=tile, split_k=split))
            ws = torch.empty(max(p.info().workspace_bytes, 4), dtype=torch.uint8, device="cuda")
            C = torch.full((M, N), float("nan"), device="cuda")
            note(f"tile {tile} split {split}: {p.describe()}")
            tcg.gemm_run_ex(p, Ad, Bd, C, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(C.cpu().numpy(), want), (tile, split)


def test_autotune_picks_caches_and_replays(tcg):
    tcg.gemm_tune_cache_clear()
    M, N, K = 256, 512, 8192  # few tiles, long K: splits are candidates
    w = gw.custom(M, N, K, BF16, F32, EPI_NONE, gw.INT4, seed=91)
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(16 * M * N, dtype=torch.float32, device="cuda")
    desc = tcg.make_desc(M, N, K, BF16, F32, EPI_NONE, tcg.FLAG_SPLIT_K)
    note("autotune 256x512x8192")
    p = tcg.gemm_autotune(desc, Ad, Bd, C, workspace=ws)
    note(f"chosen: {p.describe()}")
    assert tcg.gemm_tune_cache_size() == 1
    # the tuned plan computes the exact result
    C.fill_(float("nan"))
    tcg.gemm_run_ex(p, Ad, Bd, C, workspace=ws)
    torch.cuda.synchronize()
    check_against_oracle(w, A, B, C.cpu().reshape(1, M, N))
    # gemm_plan with GEMM_FLAG_TUNED returns the same choice
    q = tcg.gemm_plan(tcg.make_desc(M, N, K, BF16, F32, EPI_NONE, tcg.FLAG_SPLIT_K | tcg.FLAG_TUNED))
    assert (q.info().tile_id, q.info().split_k) == (p.info().tile_id, p.info().split_k)
    # without a workspace no split is a candidate
    tcg.gemm_tune_cache_clear()
    p1 = tcg.gemm_autotune(desc, Ad, Bd, C)
    assert p1.info().split_k == 1
    tcg.gemm_tune_cache_clear()


def test_matmul_tune_within_tolerance(tcg):
    tcg.gemm_tune_cache_clear()
    w = gw.custom(512, 1024, 2048, BF16, BF16, EPI_RELU, gw.NORMAL, seed=92)
    A, B = gw.make_inputs(w)
    note("matmul tune=True 512x1024x2048")
    C = tcg.matmul(A.cuda(), B.cuda(), relu=True, tune=True)
    C2 = tcg.matmul(A.cuda(), B.cuda(), relu=True, tune=True)  # cached plan: same bits
    torch.cuda.synchronize()
    assert tcg.gemm_tune_cache_size() == 1
    assert np.array_equal(as_bits(C.cpu()), as_bits(C2.cpu()))
    check_against_oracle(w, A, B, C.cpu().reshape(1, w.M, w.N))
    tcg.gemm_tune_cache_clear()


def test_matmul_tune_on_a_raw_stream_never_keeps_a_split_plan(tcg):
    """On a raw stream handle no workspace can be kept alive, so the run
    cannot split K; tune=True there must tune among unsplit plans only and
    run, on the first call and on the cached plan (a long-K, few-tile shape
    where splits would otherwise be candidates)."""
    tcg.gemm_tune_cache_clear()
    w = gw.custom(256, 512, 8192, BF16, F32, EPI_NONE, gw.INT4, seed=93)
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    raw = torch.cuda.current_stream().cuda_stream
    note("matmul tune=True on a raw stream, 256x512x8192")
    C1 = tcg.matmul(Ad, Bd, out_dtype=torch.float32, tune=True, stream=raw)
    C2 = tcg.matmul(Ad, Bd, out_dtype=torch.float32, tune=True, stream=raw)
    torch.cuda.synchronize()
    check_against_oracle(w, A, B, C1.cpu().reshape(1, w.M, w.N))
    assert np.array_equal(as_bits(C1.cpu()), as_bits(C2.cpu()))
    tcg.gemm_tune_cache_clear()


def test_autotune_considers_the_planners_split_tail(tcg):
    """4608^3 with split K allowed: the planner's own plan splits K for its
    last rows only; the autotuner times it with the tile candidates, and
    whatever wins is exact on integer inputs and replayed by
    GEMM_FLAG_TUNED (split 0 in the cache stands for the tail plan)."""
    tcg.gemm_tune_cache_clear()
    M = N = K = 4608
    w = gw.custom(M, N, K, BF16, F32, EPI_RELU, gw.INT4, seed=94)
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    desc = tcg.make_desc(M, N, K, BF16, F32, EPI_RELU, tcg.FLAG_SPLIT_K)
    planner = tcg.gemm_plan(desc).info()
    assert planner.tail_rows > 0
    ws = torch.empty(max(planner.workspace_bytes, 16 * M * N * 4) // 4, dtype=torch.float32,
                     device="cuda")
    p = tcg.gemm_autotune(desc, Ad, Bd, C, workspace=ws)
    i = p.info()
    note(f"4608^3 tuned: {p.describe()}")
    q = tcg.gemm_plan(tcg.make_desc(M, N, K, BF16, F32, EPI_RELU,
                                    tcg.FLAG_SPLIT_K | tcg.FLAG_TUNED)).info()
    assert (q.tile_id, q.split_k, q.tail_rows) == (i.tile_id, i.split_k, i.tail_rows)
    C.fill_(float("nan"))
    tcg.gemm_run_ex(p, Ad, Bd, C, workspace=ws)
    torch.cuda.synchronize()
    bi, ii, jj = gw.sample_indices(M, N, 4096, 95)
    want, _ = oracle.gemm_sampled(A, B, M, N, K, BF16, F32, EPI_RELU, bi, ii, jj)
    assert np.array_equal(C.cpu().numpy()[ii, jj], want)
    tcg.gemm_tune_cache_clear()


def test_a_restricted_search_answers_without_caching(tcg):
    """A description naming a tile or a split restricts the candidates to it,
    and its winner is returned but not cached (a later GEMM_FLAG_TUNED plan
    must not replay a partial search)."""
    tcg.gemm_tune_cache_clear()
    M, N, K = 256, 512, 8192
    w = gw.custom(M, N, K, BF16, F32, EPI_NONE, gw.INT4, seed=93)
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(16 * M * N, dtype=torch.float32, device="cuda")
    note("autotune restricted to tile 2")
    p = tcg.gemm_autotune(tcg.make_desc(M, N, K, BF16, F32, EPI_NONE, tcg.FLAG_SPLIT_K, tile=2),
                          Ad, Bd, C, workspace=ws)
    assert p.info().tile_id == 2
    assert tcg.gemm_tune_cache_size() == 0
    note("autotune restricted to 3 ranges")
    p3 = tcg.gemm_autotune(tcg.make_desc(M, N, K, BF16, F32, EPI_NONE, 0, split_k=3),
                           Ad, Bd, C, workspace=ws)
    assert p3.info().split_k == 3
    assert tcg.gemm_tune_cache_size() == 0
    C.fill_(float("nan"))
    tcg.gemm_run_ex(p3, Ad, Bd, C, workspace=ws)
    torch.cuda.synchronize()
    check_against_oracle(w, A, B, C.cpu().reshape(1, M, N))


def _tune_cases(n=24, seed=20261206):
    import random
    rng = random.Random(seed)
    out = []
    for i in range(n):
        in_dtype = rng.choice([F16, BF16, gw.FP8])
        out_dtype = rng.choice([F32, F16, BF16])
        M, N, K = rng.randint(1, 1500), rng.randint(1, 1500), rng.randint(1, 3000)
        epi = rng.choice([0, 1, 2, 3, 4, 5])
        bias = rng.random() < 0.3
        dist = gw.INT4 if (rng.random() < 0.4 and epi in (0, 1) and not bias) else gw.NORMAL
        out.append((i, M, N, K, in_dtype, out_dtype, epi, bias, dist))
    return out


@pytest.mark.parametrize("case", _tune_cases(), ids=lambda c: f"tune{c[0]}")
def test_random_problem_tuned_then_replayed_matches_the_oracle(tcg, case):
    """gemm_autotune with split K allowed and a workspace, then the cached
    choice through GEMM_FLAG_TUNED, every output against the oracle."""
    i, M, N, K, in_dtype, out_dtype, epi, bias, dist = case
    w = gw.custom(M, N, K, in_dtype, out_dtype, epi, dist, seed=9000 + i)
    A, B = gw.make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    b = gw.draw_bias(N, gw.NORMAL, seed=9500 + i) if bias else None
    bd = b.cuda() if bias else None
    flags = tcg.FLAG_SPLIT_K | (tcg.FLAG_BIAS if bias else 0)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    C = torch.empty((M, N), dtype=gw.TORCH_DTYPE[out_dtype], device="cuda")
    tcg.gemm_autotune(tcg.make_desc(M, N, K, in_dtype, out_dtype, epi, flags), Ad, Bd, C, bias=bd,
                      workspace=ws)
    p = tcg.gemm_plan(tcg.make_desc(M, N, K, in_dtype, out_dtype, epi, flags | tcg.FLAG_TUNED))
    note(f"tuned {w.name}: {p.describe()}")
    C.fill_(float("nan"))
    tcg.gemm_run_ex(p, Ad, Bd, C, bias=bd, workspace=ws if p.info().workspace_bytes else None)
    torch.cuda.synchronize()
    check_against_oracle(w, A, B, C.cpu().reshape(1, M, N), bias=b)
