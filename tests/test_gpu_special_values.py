"""NaN, infinities and out-of-range outputs through every output path.

The readings these tests check, all from the page "gizml:tile":
- Tile.relu is max(x, 0) and Tile.maximum returns the operand that is not a
  NaN, so relu(NaN) = +0 (and relu(-Inf) = +0, relu(+Inf) = +Inf);
- Tile.to rounds to the storage type as a store and a reload give: round to
  nearest even, so an fp32 value past a 16-bit type's largest finite value
  (by at least half an ulp) becomes +-Inf, and a NaN stays a NaN;
- without an activation, NaN and +-Inf pass through unchanged.

Inputs are small integers (every finite sum exact in fp32, so one correct
result) with planted special values:
- row 1 of A holds a NaN: the whole row of A.B is NaN;
- row 2 holds +Inf: +-Inf where B's matching row is non-zero, NaN where it
  is zero (Inf * 0);
- row 3 holds -Inf and +Inf: NaN wherever both B entries share a sign;
- column 4 of B holds +Inf;
- rows 5 and 6 of A are +250 and -250 everywhere and column 6 of B is 4
  everywhere: C[5, 6] = 1000 K and C[6, 6] = -1000 K, past fp16's 65504
  for every K used here (the exact sums stay below 2^24);
- with bf16 operands, row 7 of A is 2^127 (1 + 127/128), 2^119, 2^118, then
  zeros, and B's rows 0-2 are 1 in column 8 and 0 elsewhere: C[7, 8] is
  finite in fp32 (all three terms positive, exact in any order) but rounds
  to +Inf in bf16; row 8 is its negative (-Inf, and +0 under relu).
Each infinite or NaN result is the same for every order of the sum (the
terms that make it are all of one sign or the NaN comes from one product),
so the GPU must equal the oracle: same NaN positions, equal values
elsewhere, and +0 (sign bit clear) where relu meets a NaN.

Paths: the 256 x 256 tile with 16-byte copies, the element-copy path
(K and N not multiples of 8), the persistent short-K kernel, a split-K plan
(the reduction kernel's relu and rounding), and the general epilogue form
(a zero bias row selects it: its relu and rounding are separate code).
"""
import numpy as np
import pytest
import torch

import gemm_workloads as gw
import oracle
from gemm_workloads import BF16, EPI_NONE, EPI_RELU, F16, F32
from gpu_helpers import note, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    return t


# name: (M, N, K, tile, split_k, bias)
PATHS = {
    "tile1_16byte": (300, 264, 256, 1, 0, False),
    "element_copy": (130, 77, 201, 3, 0, False),
    "shortk_tile11": (1000, 288, 96, 11, 0, False),
    "split_k3": (200, 136, 768, 3, 3, False),
    "general_epilogue": (300, 264, 256, 1, 0, True),
}


def special_inputs(M, N, K, in_dtype, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(-4, 5, (M, K)).astype(np.float32)
    b = rng.integers(-4, 5, (K, N)).astype(np.float32)
    a[1, 5] = np.nan
    a[2, 7] = np.inf
    a[3, 9], a[3, 10] = -np.inf, np.inf
    b[11, 4] = np.inf
    a[5, :] = 250.0
    a[6, :] = -250.0
    b[:, 6] = 4.0
    if in_dtype == BF16:
        a[7, :] = 0.0
        a[7, 0] = np.ldexp(1.0 + 127.0 / 128.0, 127)
        a[7, 1] = np.ldexp(1.0, 119)
        a[7, 2] = np.ldexp(1.0, 118)
        a[8, :] = -a[7, :]
        b[0:3, :] = 0.0
        b[0:3, 8] = 1.0
    dt = gw.TORCH_DTYPE[in_dtype]
    return torch.from_numpy(a).to(dt), torch.from_numpy(b).to(dt)


def compare(got, want, epi, name):
    """Same NaN positions, equal values elsewhere (+0 == -0), and +0 where
    relu meets a NaN."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    bad = np.argwhere(gn != wn)
    assert bad.size == 0, f"{name}: NaN positions differ at {bad[:5].tolist()}"
    ok = ~wn
    diff = np.argwhere(ok & (got != want))
    assert diff.size == 0, (f"{name}: {len(diff)} values differ, first at {diff[:3].tolist()}: "
                            f"got {[got[tuple(i)] for i in diff[:3]]}, "
                            f"want {[want[tuple(i)] for i in diff[:3]]}")
    if epi == EPI_RELU:
        assert not np.any(np.signbit(got[1, :])), f"{name}: relu(NaN) must be +0"


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("in_dtype", [F16, BF16])
@pytest.mark.parametrize("out_dtype", [F32, F16, BF16])
@pytest.mark.parametrize("epi", [EPI_NONE, EPI_RELU])
def test_special_values_match_the_oracle(tcg, path, in_dtype, out_dtype, epi):
    M, N, K, tile, split, with_bias = PATHS[path]
    w = gw.custom(M, N, K, in_dtype, out_dtype, epi, gw.INT4, seed=0,
                  name=f"special_{path}")
    A, B = special_inputs(M, N, K, in_dtype, seed=M + N + K)
    bias = torch.zeros(N, dtype=torch.float32) if with_bias else None
    C, _, p = run(tcg, A, B, w, tile=tile, split_k=split, bias=bias)
    info = p.info()
    assert info.tile_id == tile
    if path == "tile1_16byte":
        assert info.vec16 == 1
    if path == "element_copy":
        assert info.vec16 == 0
    if split:
        assert info.split_k == split
    Cref = oracle.gemm(A, B, M, N, K, in_dtype, out_dtype, epi,
                       bias=None if bias is None else bias.numpy())
    want = oracle.to_float(out_dtype, Cref)[0]
    got = C.float().numpy()[0]
    note(f"{path}: NaN {int(np.isnan(want).sum())}, +-Inf {int(np.isinf(want).sum())} "
         f"outputs expected")
    # the planted cases really occur in the expected output
    if epi == EPI_NONE:
        assert np.isnan(want[1]).all() and np.isinf(want).any()
    else:
        # relu(NaN) = +0: the NaN row is all zeros, and no NaN is left
        assert np.all(want[1] == 0) and not np.isnan(want).any()
        assert np.isinf(want).any()
    if out_dtype == F16 and epi == EPI_NONE:
        assert np.isinf(want[5, 6]) and np.isinf(want[6, 6])
    if in_dtype == BF16 and out_dtype == BF16:
        assert want[7, 8] == np.inf
        assert (want[8, 8] == -np.inf) if epi == EPI_NONE else (want[8, 8] == 0)
    if in_dtype == BF16 and out_dtype == F32:
        assert np.isfinite(want[7, 8]) and want[7, 8] > 3.39e38
    compare(got, want, epi, f"{path} in={in_dtype} out={out_dtype} epi={epi}")


# (name, input type, output type, a, b, K): every value exact, so one result.
SUBNORMAL = [
    ("fp16 subnormal A", F16, F32, 2.0 ** -20, 2.0 ** 10, 64),
    ("fp16 subnormal A and B", F16, F32, 2.0 ** -20, 2.0 ** -16, 64),
    ("fp16 subnormal output", F16, F16, 2.0 ** -14, 2.0 ** -10, 64),
    ("bf16 subnormal A", BF16, F32, 2.0 ** -130, 2.0 ** 100, 64),
    ("fp32 subnormal output", BF16, F32, 2.0 ** -70, 2.0 ** -70, 64),
    ("bf16 subnormal output", BF16, BF16, 2.0 ** -70, 2.0 ** -65, 64),
    ("fp8 subnormal A", gw.FP8, F32, 2.0 ** -8, 2.0, 128),
    ("fp8 subnormal A and B", gw.FP8, F32, 2.0 ** -8, 2.0 ** -9, 128),
]


@pytest.mark.parametrize("name,in_dtype,out_dtype,a,b,K", SUBNORMAL, ids=[c[0] for c in SUBNORMAL])
def test_subnormal_operands_and_outputs_are_kept(tcg, name, in_dtype, out_dtype, a, b, K):
    """Subnormal operands and subnormal results are values like any other
    (gizml:tile, Tile.to: the value a store and a load of the type give): the
    MFMA and the epilogue keep them, staged and unstaged, bit for bit equal
    to the oracle's."""
    M = N = 64
    tdt = gw.TORCH_DTYPE[in_dtype]
    A = torch.full((M, K), a, dtype=torch.float32)
    A[::2] *= 3.0  # two row values, both still exact
    A, B = A.to(tdt), torch.full((K, N), b, dtype=torch.float32).to(tdt)
    want = oracle.gemm(A, B, M, N, K, in_dtype, out_dtype, EPI_NONE).reshape(M, N)
    wbits = want.view(np.int32) if out_dtype == F32 else want.view(np.int16)
    for flags in (0, tcg.FLAG_UNSTAGED):
        w = gw.custom(M, N, K, in_dtype, out_dtype, EPI_NONE, gw.NORMAL, seed=0)
        C, _, p = run(tcg, A, B, w, flags=flags)
        note(f"{name}: {p.describe()}")
        got = C.reshape(M, N).view(torch.int32 if out_dtype == F32 else torch.int16).numpy()
        assert np.array_equal(got, wbits), (name, flags)
    # the case is what its name says
    y = oracle.to_float(out_dtype, want)[1, 0]
    tiny = {F32: 2.0 ** -126, F16: 2.0 ** -14, BF16: 2.0 ** -126}[out_dtype]
    if "output" in name:
        assert 0 < y < tiny, (name, y)
