"""Pins for the CPU oracle, checked against things other than itself.

Each test ties one part of the oracle to the pages or to mathematics:
library conversions (numpy's binary16, torch's bfloat16), hand-derived
rounding cases and hand-worked products (tests/golden), exact integer
arithmetic, closed forms, a brute-force fp32 emulation written in Python,
the fp32 recursive-summation error bound, and the k order the fold of the
page "gizml:tile" fixes.  A plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a different sum order, a wrong
rounding) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, EPI_NONE, EPI_RELU, F16, F32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16_bits(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def bf16_bits(x):
    t = torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_of(dtype, x):
    return f16_bits(x) if dtype == F16 else bf16_bits(x)


def values_of(dtype, bits):
    """Library decode (numpy binary16 / torch bfloat16) of 16-bit patterns."""
    bits = np.asarray(bits, np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()


# --------------------------------------------------------------------------
# conversions
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_decode_every_pattern_matches_library(dtype):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(dtype, pats)
    ref = values_of(dtype, pats)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _encode_inputs(seed=0):
    rng = np.random.default_rng(seed)
    # wide exponent spread, both signs, plus values on exact halfway points
    mags = np.exp2(rng.uniform(-30, 20, 200000)).astype(np.float32)
    vals = mags * rng.choice([-1.0, 1.0], mags.size).astype(np.float32)
    u = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    rand_bits = u.view(np.float32)
    halfway_f16 = (rng.integers(0, 2**16, 20000).astype(np.uint32) << 13 | 0x1000).astype(np.uint32)
    halfway_bf16 = (rng.integers(0, 2**16, 20000).astype(np.uint32) << 16 | 0x8000).astype(np.uint32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.996, 65520, 1e-8, 2**-24,
                         2**-25, 3 * 2**-25], np.float32)
    return np.concatenate([vals, rand_bits, halfway_f16.view(np.float32),
                           halfway_bf16.view(np.float32), specials, _nan_inputs()]).astype(np.float32)


def _nan_inputs():
    # the default quiet NaN of both signs, quiet NaNs with low payload bits,
    # and signalling NaNs (quiet bit clear, payload nonzero)
    return np.array([0x7fc00000, 0xffc00000, 0x7fc00001, 0x7f800001, 0xff800001, 0x7fa00000,
                     0x7f802000], np.uint32).view(np.float32)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_encode_rne_matches_library(dtype):
    x = _encode_inputs(1 + dtype)
    got = oracle.encode(dtype, x)
    ref = bits_of(dtype, x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN (payload not compared)
    assert np.all(np.isnan(values_of(dtype, got[nan])))


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_encode_gives_quiet_nans(dtype):
    """A NaN, quiet or signalling, converts to a quiet NaN of the narrower
    format (IEEE 754, conversion of a NaN: the result is a quiet NaN), whatever
    payload bits survive: exponent all ones, fraction nonzero, and the
    fraction's top bit set (0x0200 in binary16, 0x0040 in bfloat16)."""
    got = oracle.encode(dtype, _nan_inputs()).astype(np.uint32)
    exp_mask, quiet = (0x7c00, 0x0200) if dtype == F16 else (0x7f80, 0x0040)
    frac_mask = 0x7fff & ~exp_mask
    assert np.all(got & exp_mask == exp_mask), [hex(v) for v in got]
    assert np.all(got & frac_mask != 0), [hex(v) for v in got]
    assert np.all(got & quiet != 0), [hex(v) for v in got]


def test_rounding_golden_cases():
    path = os.path.join(GOLDEN, "rounding.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        dt, xin, want = line.split()[:3]
        dtype = F16 if dt == "f16" else BF16
        x = np.array([int(xin, 16)], np.uint32).view(np.float32)
        got = int(oracle.encode(dtype, x)[0])
        assert got == int(want, 16), (line, hex(got))
        n += 1
    assert n >= 20


# --------------------------------------------------------------------------
# hand-worked products
def _read_golden_gemm():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "small_gemm.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        tag, *rest = line.split()
        if tag == "case":
            cur = {"name": rest[0], "A": [], "B": [], "relu": [], "none": []}
        elif tag == "shape":
            cur["shape"] = tuple(int(v) for v in rest)
        elif tag in ("A", "B", "relu", "none"):
            cur[tag].append([float(v) for v in rest])
        elif tag == "end":
            cases.append(cur)
    return cases


@pytest.mark.parametrize("in_dtype", [F16, BF16])
@pytest.mark.parametrize("out_dtype", [F32, F16, BF16])
def test_hand_worked_products(in_dtype, out_dtype):
    cases = _read_golden_gemm()
    assert len(cases) >= 3
    for c in cases:
        M, N, K = c["shape"]
        A = bits_of(in_dtype, np.array(c["A"], np.float32))
        B = bits_of(in_dtype, np.array(c["B"], np.float32))
        for epi, key in ((EPI_RELU, "relu"), (EPI_NONE, "none")):
            C = oracle.gemm(A, B, M, N, K, in_dtype, out_dtype, epi)
            got = oracle.to_float(out_dtype, C)[0]
            want = np.array(c[key], np.float32)
            assert np.array_equal(got, want), (c["name"], key, got, want)
            # relu never leaves a negative zero
            if epi == EPI_RELU:
                assert not np.any(np.signbit(got)), c["name"]


# --------------------------------------------------------------------------
# exact integer arithmetic and closed forms
def _ints(rng, shape, lo=-4, hi=4):
    return rng.integers(lo, hi + 1, shape).astype(np.float32)


@pytest.mark.parametrize("in_dtype", [F16, BF16])
def test_integer_inputs_exact(in_dtype):
    rng = np.random.default_rng(7)
    M, N, K = 37, 29, 256
    a, b = _ints(rng, (M, K)), _ints(rng, (K, N))
    exact = a.astype(np.int64) @ b.astype(np.int64)  # |partial sums| <= 256*16 < 2^24
    C = oracle.gemm(bits_of(in_dtype, a), bits_of(in_dtype, b), M, N, K, in_dtype, F32,
                    EPI_NONE)[0]
    assert np.array_equal(C, exact.astype(np.float32))
    C = oracle.gemm(bits_of(in_dtype, a), bits_of(in_dtype, b), M, N, K, in_dtype, F32,
                    EPI_RELU)[0]
    assert np.array_equal(C, np.maximum(exact, 0).astype(np.float32))


def test_identity_operands_return_the_other_operand():
    rng = np.random.default_rng(8)
    n, p = 24, 19
    B = rng.standard_normal((n, p)).astype(np.float32)
    A = rng.standard_normal((p, n)).astype(np.float32)
    eye = np.eye(n, dtype=np.float32)
    for dt in (F16, BF16):
        Bb, Ab = bits_of(dt, B), bits_of(dt, A)
        # I . B = B exactly (a non-square, non-symmetric B: a transposed operand fails)
        C = oracle.gemm(bits_of(dt, eye), Bb, n, p, n, dt, dt, EPI_NONE)[0]
        assert np.array_equal(C, Bb)
        # A . I = A; relu keeps only the positive entries, negatives become +0
        C = oracle.gemm(Ab, bits_of(dt, np.eye(n, dtype=np.float32)), p, n, n, dt, F32,
                        EPI_RELU)[0]
        assert np.array_equal(C, np.maximum(values_of(dt, Ab), 0.0))
        assert not np.any(np.signbit(C))


def test_all_ones_gives_k():
    for K in (1, 7, 255, 2048):
        C = oracle.gemm(f16_bits(np.ones((3, K))), f16_bits(np.ones((K, 5))), 3, 5, K, F16, F32,
                        EPI_NONE)
        assert np.all(C == K)


def test_integer_checksum_and_transpose_identity():
    rng = np.random.default_rng(9)
    M, N, K = 45, 33, 70
    a, b = _ints(rng, (M, K)), _ints(rng, (K, N))
    C = oracle.gemm(f16_bits(a), f16_bits(b), M, N, K, F16, F32, EPI_NONE)[0]
    # sum_ij C_ij = (1^T A)(B 1), in int64
    lhs = int(C.astype(np.int64).sum())
    rhs = int(a.astype(np.int64).sum(0) @ b.astype(np.int64).sum(1))
    assert lhs == rhs
    # relu(A.B)^T = relu(B^T A^T)
    C1 = oracle.gemm(f16_bits(a), f16_bits(b), M, N, K, F16, F32, EPI_RELU)[0]
    C2 = oracle.gemm(f16_bits(b.T.copy()), f16_bits(a.T.copy()), N, M, K, F16, F32, EPI_RELU)[0]
    assert np.array_equal(C1.T, C2)


def test_k_zero_gives_positive_zero():
    for out in (F32, F16, BF16):
        for epi in (EPI_NONE, EPI_RELU):
            C = oracle.gemm(np.zeros(0, np.uint16), np.zeros(0, np.uint16), 3, 4, 0, F16, out, epi)
            assert C.shape == (1, 3, 4)
            assert np.all(C.view(np.uint32 if out == F32 else np.uint16) == 0)


def test_k_zero_applies_the_epilogue_to_zero():
    """K = 0 leaves the zero accumulator, and the epilogue still runs on it
    (page "gizml:tile": Program.zeros, then the epilogue): sigmoid(0) = 1/2,
    tanh(0) = gelu(0) = 0, and with a bias row, act(bias[j])."""
    z = np.zeros(0, np.uint16)
    C = oracle.gemm(z, z, 2, 3, 0, F16, F32, oracle.EPI_SIGMOID)
    assert np.all(C == 0.5)
    for epi in (oracle.EPI_TANH, oracle.EPI_GELU, oracle.EPI_GELU_ERF):
        C = oracle.gemm(z, z, 2, 3, 0, BF16, F32, epi)
        assert np.all(C.view(np.uint32) == 0)
    bias = np.array([-1.5, 0.25, 3.0], np.float32)
    C = oracle.gemm(z, z, 2, 3, 0, F16, F32, EPI_RELU, bias=bias)
    assert np.array_equal(C[0], np.array([[0.0, 0.25, 3.0]] * 2, np.float32))
    C = oracle.gemm(z, z, 2, 3, 0, F16, F32, oracle.EPI_SIGMOID, bias=bias)
    assert np.allclose(C[0, 0], 1.0 / (1.0 + np.exp(-bias.astype(np.float64))), rtol=1e-7, atol=0)


# --------------------------------------------------------------------------
# order and fp32 semantics
def test_products_round_to_fp32_before_the_sum():
    """Tile.dot in F32 (page "gizml:tile"): each product is an fp32 value
    before it joins the sum, so a product beyond fp32's range is infinite even
    where the partial sum would cancel it, and a product below half of the
    smallest subnormal is zero.  A fused multiply-add, or a wider accumulator,
    gives a finite result in the first case and 2^-148 in the second."""
    # -2^127 * 1 + 2^127 * 2: fl32(2^128) = +Inf, so the sum is +Inf (exact: 2^127)
    a = np.array([[-(2.0**127), 2.0**127]], np.float32)
    b = np.array([[1.0], [2.0]], np.float32)
    C = oracle.gemm(bf16_bits(a), bf16_bits(b), 1, 1, 2, BF16, F32, EPI_NONE)
    assert np.isposinf(C[0, 0, 0])
    # 2^-75 * 2^-74 = 2^-149 (the smallest subnormal), then 2^-75 * 2^-75 =
    # 2^-150 rounds to 0 (a tie, to even), so the sum stays 2^-149
    a = np.array([[2.0**-75, 2.0**-75]], np.float32)
    b = np.array([[2.0**-74], [2.0**-75]], np.float32)
    C = oracle.gemm(bf16_bits(a), bf16_bits(b), 1, 1, 2, BF16, F32, EPI_NONE)
    assert C.view(np.uint32)[0, 0, 0] == 1


def test_fold_runs_k_ascending_in_fp32():
    # bf16 holds 2^24 exactly.  In fp32, k ascending: 2^24 + 1 -> 2^24 (tie to
    # even), + 1 -> 2^24, - 2^24 -> 0.  The exact sum is 2; k descending gives 2.
    a = np.array([[2.0**24, 1.0, 1.0, -(2.0**24)]], np.float32)
    b = np.ones((4, 1), np.float32)
    C = oracle.gemm(bf16_bits(a), bf16_bits(b), 1, 1, 4, BF16, F32, EPI_NONE)
    assert C[0, 0, 0] == 0.0
    Y64, _ = oracle.gemm_f64(bf16_bits(a), bf16_bits(b), 1, 1, 4, BF16)
    assert Y64[0, 0, 0] == 2.0
    C = oracle.gemm(bf16_bits(a[:, ::-1].copy()), bf16_bits(b), 1, 1, 4, BF16, F32, EPI_NONE)
    assert C[0, 0, 0] == 2.0


def _emulate(a, b, epi, out_dtype):
    """Brute force in Python: numpy float32 scalars, k ascending."""
    M, K = a.shape
    N = b.shape[1]
    y = np.zeros((M, N), np.float32)
    for i in range(M):
        for j in range(N):
            acc = np.float32(0.0)
            for k in range(K):
                acc = np.float32(acc + np.float32(a[i, k] * b[k, j]))
            if epi == EPI_RELU:
                acc = acc if acc > 0 else np.float32(0.0)
            y[i, j] = acc
    if out_dtype == F32:
        return y
    return bits_of(out_dtype, y)


SHAPES = [(1, 1, 1), (2, 3, 7), (3, 2, 16), (7, 17, 31), (16, 16, 33), (5, 65, 64), (17, 3, 65)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("in_dtype,out_dtype", [(F16, F32), (BF16, BF16), (F16, F16)])
def test_brute_force_tiny(M, N, K, in_dtype, out_dtype):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    a = values_of(in_dtype, bits_of(in_dtype, rng.standard_normal((M, K)) * 3))
    b = values_of(in_dtype, bits_of(in_dtype, rng.standard_normal((K, N))))
    for epi in (EPI_NONE, EPI_RELU):
        want = _emulate(a, b, epi, out_dtype)
        got = oracle.gemm(bits_of(in_dtype, a), bits_of(in_dtype, b), M, N, K, in_dtype,
                          out_dtype, epi)[0]
        assert np.array_equal(got.view(np.uint32 if out_dtype == F32 else np.uint16),
                              want.view(np.uint32 if out_dtype == F32 else np.uint16))


@pytest.mark.parametrize("in_dtype", [F16, BF16])
def test_fp32_within_recursive_summation_bound(in_dtype):
    rng = np.random.default_rng(11)
    M, N, K = 23, 31, 1000
    A = bits_of(in_dtype, rng.standard_normal((M, K)))
    B = bits_of(in_dtype, rng.standard_normal((K, N)))
    _, Y = oracle.gemm(A, B, M, N, K, in_dtype, F32, EPI_NONE, want_y=True)
    Y64, S64 = oracle.gemm_f64(A, B, M, N, K, in_dtype)
    u = 2.0**-24
    gamma = K * u / (1 - K * u)
    err = np.abs(Y.astype(np.float64) - Y64)
    assert np.all(err <= gamma * S64 + 1e-300)
    # and it is not trivially zero: fp32 really rounds somewhere
    assert np.any(err > 0)
    # the f64 twin is the exact product-sum to within double rounding
    exact = values_of(in_dtype, A).astype(np.float64) @ values_of(in_dtype, B).astype(np.float64)
    assert np.allclose(Y64[0], exact, rtol=0, atol=1e-9)


def test_relu_of_nan_and_negative_zero():
    # A row with a NaN gives NaN without the epilogue and +0 with relu
    # (Tile.maximum returns the operand that is not NaN).
    a = np.array([[np.nan, 1.0], [-0.0, 0.0]], np.float32)
    b = np.array([[1.0], [1.0]], np.float32)
    for dt in (F16, BF16):
        C = oracle.gemm(bits_of(dt, a), bits_of(dt, b), 2, 1, 2, dt, F32, EPI_NONE)[0]
        assert np.isnan(C[0, 0])
        C = oracle.gemm(bits_of(dt, a), bits_of(dt, b), 2, 1, 2, dt, F32, EPI_RELU)[0]
        assert C[0, 0] == 0.0 and not np.signbit(C[0, 0])
        assert C[1, 0] == 0.0 and not np.signbit(C[1, 0])
    # -x * x sums to a negative value: relu clamps to +0; without it stays negative
    a = np.array([[-2.0, -3.0]], np.float32)
    C = oracle.gemm(f16_bits(a), f16_bits(b), 1, 1, 2, F16, F32, EPI_NONE)[0]
    assert C[0, 0] == -5.0


def test_batch_items_of_c_follow_their_stride():
    """Item b of C starts at b * stride_c; the elements between items are
    left as they were."""
    rng = np.random.default_rng(14)
    M, N, K, batch, sc = 4, 5, 6, 3, 4 * 5 + 9
    A = f16_bits(rng.standard_normal(batch * M * K))
    B = f16_bits(rng.standard_normal(batch * K * N))
    want = oracle.gemm(A, B, M, N, K, F16, F16, EPI_NONE, batch=batch)
    flat = oracle.gemm(A, B, M, N, K, F16, F16, EPI_NONE, batch=batch, stride_c=sc)
    assert flat.shape == ((batch - 1) * sc + M * N,)
    for b_ in range(batch):
        assert np.array_equal(flat[b_ * sc:b_ * sc + M * N].reshape(M, N), want[b_])
        if b_ + 1 < batch:
            assert np.all(flat[b_ * sc + M * N:(b_ + 1) * sc] == oracle.C_SENTINEL16)


def test_batch_items_follow_their_strides():
    rng = np.random.default_rng(12)
    M, N, K, batch = 5, 6, 9, 3
    sa, sb = M * K + 7, K * N + 3  # padding between items
    Aall = rng.standard_normal(batch * sa).astype(np.float32)
    Ball = rng.standard_normal(batch * sb).astype(np.float32)
    C = oracle.gemm(f16_bits(Aall), f16_bits(Ball), M, N, K, F16, F32, EPI_RELU, batch=batch,
                    stride_a=sa, stride_b=sb)
    for b_ in range(batch):
        a = values_of(F16, f16_bits(Aall[b_ * sa:b_ * sa + M * K].reshape(M, K)))
        b = values_of(F16, f16_bits(Ball[b_ * sb:b_ * sb + K * N].reshape(K, N)))
        assert np.array_equal(C[b_], _emulate(a, b, EPI_RELU, F32))


@pytest.mark.parametrize("in_dtype,out_dtype", [(F16, F32), (BF16, BF16)])
def test_sampled_brute_force(in_dtype, out_dtype):
    """The sampled entry point against the Python fp32 emulation directly."""
    rng = np.random.default_rng(21 + in_dtype)
    M, N, K = 9, 11, 37
    a = values_of(in_dtype, bits_of(in_dtype, rng.standard_normal((M, K))))
    b = values_of(in_dtype, bits_of(in_dtype, rng.standard_normal((K, N))))
    ii, jj = rng.integers(0, M, 40), rng.integers(0, N, 40)
    for epi in (EPI_NONE, EPI_RELU):
        want = _emulate(a, b, epi, out_dtype)[ii, jj]
        got, _ = oracle.gemm_sampled(bits_of(in_dtype, a), bits_of(in_dtype, b), M, N, K, in_dtype,
                                     out_dtype, epi, np.zeros(40), ii, jj)
        kind = np.uint32 if out_dtype == F32 else np.uint16
        assert np.array_equal(got.view(kind), want.view(kind))


def test_sampled_equals_full():
    rng = np.random.default_rng(13)
    M, N, K = 40, 50, 77
    A = bf16_bits(rng.standard_normal((M, K)))
    B = bf16_bits(rng.standard_normal((K, N)))
    C, Y = oracle.gemm(A, B, M, N, K, BF16, BF16, EPI_RELU, want_y=True)
    ii = rng.integers(0, M, 300)
    jj = rng.integers(0, N, 300)
    out, y = oracle.gemm_sampled(A, B, M, N, K, BF16, BF16, EPI_RELU, np.zeros(300), ii, jj)
    assert np.array_equal(out, C[0, ii, jj])
    assert np.array_equal(y, Y[0, ii, jj])


def test_bad_arguments_are_rejected():
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros(4, np.uint16), np.zeros(4, np.uint16), 2, 2, 2, 3, F32, EPI_NONE)
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros(4, np.uint16), np.zeros(4, np.uint16), 2, 2, 2, F16, F32, 6)
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros(4, np.uint16), np.zeros(4, np.uint16), 2, 2, 2, F16, F32, EPI_NONE,
                    bias=np.zeros(3, np.float32))
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros(3, np.uint16), np.zeros(4, np.uint16), 2, 2, 2, F16, F32, EPI_NONE)
    # FP8 is an operand type only: an FP8 output is refused
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros(4, np.uint16), np.zeros(4, np.uint16), 2, 2, 2, F16, oracle.FP8, EPI_NONE)
    with pytest.raises(ValueError):
        oracle.gemm_sampled(np.zeros(4, np.uint16), np.zeros(4, np.uint16), 2, 2, 2, F16, oracle.FP8,
                            EPI_NONE, [0], [0], [0])


def test_workload_integer_config_is_exact_by_bound():
    # the integer workload's partial sums stay below 2^24 (one correct result)
    import gemm_workloads as gw
    w = gw.WORKLOADS["int_fp16_256"]
    assert w.K * 4 * 4 < 2**24
    A, B = gw.make_inputs(w)
    assert A.abs().max() <= 4 and B.abs().max() <= 4
    C = oracle.gemm(A, B, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue)[0]
    exact = A.double().numpy().astype(np.int64) @ B.double().numpy().astype(np.int64)
    assert np.array_equal(C, np.maximum(exact, 0).astype(np.float32))
    assert math.isclose(w.sigma_out(), math.sqrt(256) * (80 / 12), rel_tol=1e-12)


@pytest.mark.parametrize("in_dtype", [F16, BF16])
def test_f64_twin_sums_exactly_on_integers(in_dtype):
    # The fp64 twin's two outputs against int64 arithmetic: with integer
    # operands every partial sum is an integer far below 2^53, so Y64 must
    # equal A.B and S64 must equal |A|.|B| exactly (a doubled, dropped or
    # signed term in either fails).  Batch items with padding between them
    # check the strides.
    rng = np.random.default_rng(21)
    M, N, K, batch = 9, 13, 300, 2
    sa, sb = M * K + 5, K * N + 3
    Aall = rng.integers(-40, 41, batch * sa)
    Ball = rng.integers(-40, 41, batch * sb)
    Y64, S64 = oracle.gemm_f64(bits_of(in_dtype, Aall.astype(np.float32)),
                               bits_of(in_dtype, Ball.astype(np.float32)), M, N, K, in_dtype,
                               batch=batch, stride_a=sa, stride_b=sb)
    for b in range(batch):
        a = Aall[b * sa:b * sa + M * K].reshape(M, K).astype(np.int64)
        bb = Ball[b * sb:b * sb + K * N].reshape(K, N).astype(np.int64)
        assert np.array_equal(Y64[b], (a @ bb).astype(np.float64))
        assert np.array_equal(S64[b], (np.abs(a) @ np.abs(bb)).astype(np.float64))
