"""Pins of the oracle's FP8 operands (page "gizml:tile", Constants: FP8 =
9, the FP8 E4M3 storage type, read as the OCP 8-bit E4M3
format).  The decode is checked against torch's float8_e4m3fn conversion
for all 256 patterns and against hand-derived values; products and sums
against exact integer arithmetic and a brute-force fp32 emulation."""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import EPI_NONE, EPI_RELU, F16, F32, FP8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def fp8_bits(x):
    t = torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def fp8_values(bits):
    return torch.from_numpy(np.asarray(bits, np.uint8).copy()).view(torch.float8_e4m3fn).float().numpy()


def test_decode_every_pattern_matches_library():
    pats = np.arange(256, dtype=np.uint8)
    got = oracle.decode(FP8, pats)
    ref = fp8_values(pats)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.flatnonzero(nan).tolist() == [0x7F, 0xFF]
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_decode_golden_values():
    """Hand-derived from the bit layout (tests/golden/fp8_e4m3.txt)."""
    rows = []
    with open(os.path.join(GOLDEN, "fp8_e4m3.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                pat, val = line.split()
                rows.append((int(pat, 16), val))
    pats = np.array([r[0] for r in rows], np.uint8)
    got = oracle.decode(FP8, pats)
    for (p, v), g in zip(rows, got):
        if v == "nan":
            assert np.isnan(g), hex(p)
        else:
            assert g == np.float32(float.fromhex(v)) and np.signbit(g) == v.startswith("-"), hex(p)


def test_integer_products_exact():
    """Integers in [-8, 8] are exact in E4M3; |partial sums| <= 512 * 64 < 2^24."""
    rng = np.random.default_rng(21)
    M, N, K = 33, 47, 512
    a = rng.integers(-8, 9, (M, K)).astype(np.float32)
    b = rng.integers(-8, 9, (K, N)).astype(np.float32)
    exact = a.astype(np.int64) @ b.astype(np.int64)
    for epi, want in ((EPI_NONE, exact), (EPI_RELU, np.maximum(exact, 0))):
        C = oracle.gemm(fp8_bits(a), fp8_bits(b), M, N, K, FP8, F32, epi)[0]
        assert np.array_equal(C, want.astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 17), (9, 4, 64), (6, 33, 129)])
def test_brute_force_fp32_emulation(M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = fp8_values(fp8_bits(rng.standard_normal((M, K)) * 2))
    b = fp8_values(fp8_bits(rng.standard_normal((K, N))))
    y = np.zeros((M, N), np.float32)
    for i in range(M):
        for j in range(N):
            acc = np.float32(0.0)
            for k in range(K):
                acc = np.float32(acc + np.float32(a[i, k] * b[k, j]))
            y[i, j] = acc
    C = oracle.gemm(fp8_bits(a), fp8_bits(b), M, N, K, FP8, F32, EPI_NONE)[0]
    assert np.array_equal(C.view(np.uint32), y.view(np.uint32))
    C16 = oracle.gemm(fp8_bits(a), fp8_bits(b), M, N, K, FP8, F16, EPI_NONE)[0]
    assert np.array_equal(C16, y.astype(np.float16).view(np.uint16))


def test_sampled_and_f64_twin_take_fp8():
    rng = np.random.default_rng(3)
    M, N, K = 20, 30, 100
    A = fp8_bits(rng.standard_normal((M, K)))
    B = fp8_bits(rng.standard_normal((K, N)))
    C, Y = oracle.gemm(A, B, M, N, K, FP8, F32, EPI_RELU, want_y=True)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    out, Ys = oracle.gemm_sampled(A, B, M, N, K, FP8, F32, EPI_RELU, np.zeros(M * N, np.int64),
                                  ii.ravel(), jj.ravel())
    assert np.array_equal(Ys, Y.ravel())
    Y64, S64 = oracle.gemm_f64(A, B, M, N, K, FP8)
    ref = fp8_values(A).astype(np.float64) @ fp8_values(B).astype(np.float64)
    assert np.array_equal(Y64[0], ref)  # products exact in double, sums of <= 100 terms exact too
