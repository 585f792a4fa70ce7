"""A seeded sweep of random problems through the C ABI against the oracle.

Sizes from 1 to ~700 on every side (K from 0), ragged against every tile,
operands fp16, bf16 or FP8, outputs fp32, fp16 or bf16, every activation,
with and without a bias row, on the planner's choice or on an explicit tile
(the persistent short-K tile where its limits allow).  Integer inputs must
match exactly; Gaussian ones within the relative tolerance.  Larger problems
(sides up to 8192, the planner with split K allowed) are checked on sampled
outputs.
"""
import random

import pytest
import torch

import gemm_workloads as gw
from gemm_workloads import BF16, F16, F32, FP8
from gpu_helpers import check_against_oracle, check_sampled, note, run

pytestmark = pytest.mark.gpu

SIXTEEN_BIT_TILES = [1, 2, 3, 4, 5, 6, 7, 12, 13]
FP8_TILES = [8, 9, 10]


def cases(n=200, seed=20261202):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        in_dtype = rng.choice([F16, BF16, FP8])
        out_dtype = rng.choice([F32, F16, BF16])
        M = rng.choice([1, 2, 31, 33, 64, 127, 129, 255, 300, 513, 700]) if rng.random() < 0.5 else rng.randint(1, 700)
        if rng.random() < 0.3:  # a short-K, narrow-N problem
            N = rng.choice([8, 56, 96, 136, 200, 288])
            K = rng.choice([8, 16, 40, 64, 88, 96])
        else:
            N = rng.choice([1, 8, 96, 136, 256, 288, 300, 511]) if rng.random() < 0.5 else rng.randint(1, 700)
            K = rng.choice([0, 1, 8, 16, 40, 64, 96, 128, 200, 520]) if rng.random() < 0.5 else rng.randint(1, 700)
        epi = rng.choice([0, 1, 1, 2, 3, 4, 5])
        bias = rng.random() < 0.3
        dist = gw.INT4 if (rng.random() < 0.4 and epi in (0, 1) and not bias) else gw.NORMAL
        short_k_ok = (in_dtype != FP8 and 0 < K <= 96 and K % 8 == 0 and 0 < N <= 288 and N % 8 == 0
                      and epi in (0, 1) and not bias)
        r = rng.random()
        if short_k_ok and r < 0.6:
            tile = 11
        elif r < 0.45:
            tile = 0
        else:
            tile = rng.choice(FP8_TILES if in_dtype == FP8 else SIXTEEN_BIT_TILES)
        out.append((i, M, N, K, in_dtype, out_dtype, epi, bias, dist, tile))
    return out


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    return t


@pytest.mark.parametrize("case", cases(), ids=lambda c: f"case{c[0]}")
def test_random_problem_matches_the_oracle(tcg, case):
    i, M, N, K, in_dtype, out_dtype, epi, bias, dist, tile = case
    w = gw.custom(M, N, K, in_dtype, out_dtype, epi, dist, seed=1000 + i)
    A, B = gw.make_inputs(w)
    b = gw.draw_bias(N, gw.NORMAL, seed=2000 + i) if bias else None
    split = 0 if tile == 11 else (3 if i % 7 == 0 and K > 256 else 0)
    if K == 0:
        A = torch.zeros(0, dtype=A.dtype)
        B = torch.zeros(0, dtype=B.dtype)
    C, _, p = run(tcg, A, B, w, tile=tile, bias=b, split_k=split)
    if tile:
        assert p.info().tile_id == tile
    check_against_oracle(w, A, B, C, bias=b)


SENTINEL = 0x5A5A


def wide_cases(n=120, seed=20261203):
    """Batches of up to 3 items, sides up to 1200 (many ragged trips on every
    tile), the stage and split flags, operands shifted off 16-byte alignment
    (the element-copy path), and guard bands around C whose length also
    shifts C (a guard of 1 or 63 elements: the element-by-element stores)."""
    rng = random.Random(seed)
    flag_names = ["none", "stages1", "unstaged", "stages2", "split"]
    out = []
    for i in range(n):
        in_dtype = rng.choice([F16, BF16, FP8])
        out_dtype = rng.choice([F32, F16, BF16])
        batch = rng.choice([1, 1, 2, 3])
        M = rng.randint(1, 1200)
        N = rng.choice([rng.randint(1, 1200), rng.choice([8, 256, 520, 1024])])
        K = rng.choice([rng.randint(1, 1200), rng.choice([0, 64, 128, 1000, 1024])])
        epi = rng.choice([0, 1, 1, 2, 3, 4, 5])
        bias = rng.random() < 0.3
        dist = gw.INT4 if (rng.random() < 0.4 and epi in (0, 1) and not bias) else gw.NORMAL
        flag = rng.choice(flag_names)
        shift = rng.choice([0, 0, 0, 1, 3])
        tile = 0 if rng.random() < 0.5 else rng.choice(FP8_TILES if in_dtype == FP8 else
                                                         [t for t in SIXTEEN_BIT_TILES])
        guard = rng.choice([64, 64, 63, 1])
        out.append((i, batch, M, N, K, in_dtype, out_dtype, epi, bias, dist, flag, shift, tile, guard))
    return out


@pytest.mark.parametrize("case", wide_cases(), ids=lambda c: f"wide{c[0]}")
def test_wide_random_problem_matches_the_oracle(tcg, case):
    i, batch, M, N, K, in_dtype, out_dtype, epi, bias, dist, flag, shift, tile, guard = case
    w = gw.custom(M, N, K, in_dtype, out_dtype, epi, dist, seed=3000 + i, batch=batch)
    A, B = gw.make_inputs(w)
    b = gw.draw_bias(N, gw.NORMAL, seed=4000 + i) if bias else None
    flags = {"none": 0, "stages1": tcg.FLAG_FORCE_STAGES_1, "unstaged": tcg.FLAG_UNSTAGED,
             "stages2": tcg.FLAG_FORCE_STAGES_2, "split": tcg.FLAG_SPLIT_K}[flag]
    if K == 0:
        A = torch.zeros(0, dtype=A.dtype)
        B = torch.zeros(0, dtype=B.dtype)
    sentinel = SENTINEL | (SENTINEL << 16) if out_dtype == F32 else SENTINEL
    C, buf, p = run(tcg, A, B, w, flags=flags, tile=tile, bias=b, a_offset=shift, b_offset=shift,
                    guard=guard, sentinel=sentinel)
    if tile:
        assert p.info().tile_id == tile
    bits = buf.view(torch.int32 if out_dtype == F32 else torch.int16)
    assert torch.all(bits[:guard] == sentinel) and torch.all(bits[-guard:] == sentinel), "guard band written"
    check_against_oracle(w, A, B, C, bias=b)


def split_cases(n=100, seed=20261204):
    """Explicit K splits of 2 to 16 ranges (the reduction applies the bias,
    the activation and the output rounding), on any tile, batches of up to
    2 items."""
    rng = random.Random(seed)
    out = []
    for i in range(n):
        in_dtype = rng.choice([F16, BF16, FP8])
        out_dtype = rng.choice([F32, F16, BF16])
        split = rng.choice([2, 3, 4, 5, 8, 16])
        M = rng.randint(1, 600)
        N = rng.randint(1, 600)
        K = rng.randint(64 * split, 3000)
        epi = rng.choice([0, 1, 2, 3, 4, 5])
        bias = rng.random() < 0.5
        dist = gw.INT4 if (rng.random() < 0.4 and epi in (0, 1) and not bias) else gw.NORMAL
        batch = rng.choice([1, 1, 2])
        tile = 0 if rng.random() < 0.4 else rng.choice(FP8_TILES if in_dtype == FP8 else SIXTEEN_BIT_TILES)
        out.append((i, batch, M, N, K, in_dtype, out_dtype, epi, bias, dist, split, tile))
    return out


@pytest.mark.parametrize("case", split_cases(), ids=lambda c: f"split{c[0]}")
def test_split_random_problem_matches_the_oracle(tcg, case):
    i, batch, M, N, K, in_dtype, out_dtype, epi, bias, dist, split, tile = case
    w = gw.custom(M, N, K, in_dtype, out_dtype, epi, dist, seed=5000 + i, batch=batch)
    A, B = gw.make_inputs(w)
    b = gw.draw_bias(N, gw.NORMAL, seed=6000 + i) if bias else None
    C, _, p = run(tcg, A, B, w, tile=tile, bias=b, split_k=split)
    info = p.info()
    if tile:
        assert info.tile_id == tile
    # the planner keeps ranges of whole trips: at most `split` of them
    assert 1 <= info.split_k <= split
    check_against_oracle(w, A, B, C, bias=b)


def large_cases(n=40, seed=20261205):
    """Sides from 1000 to 8192 (several rounds of tiles on every tile size,
    small last rounds), the planner's plan with split K allowed on most (so
    whole-problem splits and split tails), every operand and output type and
    activation, bias rows on some."""
    rng = random.Random(seed)
    out = []
    for i in range(n):
        in_dtype = rng.choice([F16, BF16, FP8])
        out_dtype = rng.choice([F32, F16, BF16])
        M = rng.randint(1000, 8192)
        N = rng.choice([rng.randint(1000, 8192), 8 * rng.randint(125, 1024)])
        K = rng.choice([rng.randint(1, 8192), 64 * rng.randint(1, 128)])
        epi = rng.choice([0, 1, 1, 2, 3, 4, 5])
        bias = rng.random() < 0.3
        dist = gw.INT4 if (rng.random() < 0.3 and epi in (0, 1) and not bias) else gw.NORMAL
        split = rng.random() < 0.7
        out.append((i, M, N, K, in_dtype, out_dtype, epi, bias, dist, split))
    return out


@pytest.mark.parametrize("case", large_cases(), ids=lambda c: f"large{c[0]}")
def test_large_random_problem_matches_the_oracle_on_samples(tcg, case):
    i, M, N, K, in_dtype, out_dtype, epi, bias, dist, split = case
    w = gw.custom(M, N, K, in_dtype, out_dtype, epi, dist, seed=7000 + i)
    g = torch.Generator(device="cuda").manual_seed(7000 + i)
    A = gw.draw((M, K), dist, in_dtype, g)
    B = gw.draw((K, N), dist, in_dtype, g)
    b = gw.draw_bias(N, gw.NORMAL, seed=8000 + i) if bias else None
    flags = (tcg.FLAG_SPLIT_K if split else 0) | (tcg.FLAG_BIAS if bias else 0)
    p = tcg.gemm_plan(tcg.make_desc(M, N, K, in_dtype, out_dtype, epi, flags))
    note(f"large{i}: {M}x{N}x{K}: {p.describe()}")
    C = torch.full((M, N), float("nan"), dtype=gw.TORCH_DTYPE[out_dtype], device="cuda")
    wsb = p.info().workspace_bytes
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
    tcg.gemm_run_ex(p, A, B, C, bias=b.cuda() if bias else None, workspace=ws)
    torch.cuda.synchronize()
    check_sampled(w, A.cpu(), B.cpu(), C.cpu().reshape(1, M, N), count=2048, seed=i, bias=b)
