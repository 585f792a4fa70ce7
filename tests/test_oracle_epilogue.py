"""Pins of the oracle's epilogue: bias row and activations (page
"gizml:tile": Tile.add with broadcasting, Tile.relu, Tile.gelu,
Tile.geluErf, Tile.sigmoid, Tile.tanh).

Each activation is pinned to something other than the oracle's own
formula: a library routine evaluated in double precision (numpy's tanh,
scipy's expit and erfc, the last through the identity 1 + erf(x) =
erfc(-x)), a symmetry every correct implementation satisfies, or a value
fixed by the mathematics.  The bias is pinned with identity operands, where
the product is exact.
"""
import numpy as np
import pytest
from scipy import special

import oracle
from oracle import (BF16, EPI_GELU, EPI_GELU_ERF, EPI_NONE, EPI_RELU, EPI_SIGMOID, EPI_TANH, F16,
                    F32)

# fp16-exact inputs spanning the interesting range (steps of 1/64 in [-8, 8]).
X = np.arange(-512, 513, dtype=np.float32) / 64.0


def act_of(x, epi, out_dtype=F32):
    """The oracle's epilogue on the values x: C = act(1 * x) with K = 1."""
    xb = oracle.encode(F16, x).reshape(1, -1)
    one = oracle.encode(F16, np.ones(1, np.float32)).reshape(1, 1)
    C = oracle.gemm(one, xb, 1, x.size, 1, F16, out_dtype, epi)
    return oracle.to_float(out_dtype, C).reshape(-1)


def ulps(a, b):
    """Distance in fp32 units in the last place."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7fffffff), ia)
    ib = np.where(ib < 0, -(ib & 0x7fffffff), ib)
    return np.abs(ia - ib)


def test_sigmoid_is_the_logistic_function():
    got = act_of(X, EPI_SIGMOID)
    want = special.expit(X.astype(np.float64)).astype(np.float32)
    assert ulps(got, want).max() <= 1
    assert act_of(np.zeros(1, np.float32), EPI_SIGMOID)[0] == 0.5


def test_tanh_is_the_hyperbolic_tangent():
    got = act_of(X, EPI_TANH)
    want = np.tanh(X.astype(np.float64)).astype(np.float32)
    assert ulps(got, want).max() <= 1
    assert np.array_equal(got, -act_of(-X, EPI_TANH))  # odd


def test_gelu_erf_form_matches_erfc():
    got = act_of(X, EPI_GELU_ERF)
    x = X.astype(np.float64)
    want = (0.5 * x * special.erfc(-x / np.sqrt(2.0))).astype(np.float32)
    # the erf form loses relative precision where 1 + erf(x) cancels (x < -5)
    ok = X > -5
    assert ulps(got[ok], want[ok]).max() <= 2
    assert np.max(np.abs(got - want)) < 1e-6


@pytest.mark.parametrize("epi", [EPI_GELU, EPI_GELU_ERF])
def test_gelu_minus_its_mirror_is_x(epi):
    # x Phi(x) - (-x) Phi(-x) = x (1 - Phi(-x) ... ) = x, in both forms,
    # because the tanh and erf terms are odd
    got = act_of(X, epi).astype(np.float64) - act_of(-X, epi).astype(np.float64)
    assert np.max(np.abs(got - X) / np.maximum(np.abs(X), 1.0)) < 1e-6


def test_gelu_tanh_form_approximates_the_erf_form():
    # the tanh form is an approximation of x Phi(x); its error is small but
    # not zero, which pins the form and its two constants
    t = act_of(X, EPI_GELU).astype(np.float64)
    x = X.astype(np.float64)
    e = 0.5 * x * special.erfc(-x / np.sqrt(2.0))
    d = np.abs(t - e)
    assert d.max() < 1e-3
    assert d.max() > 1e-5  # a different function, not the erf form again
    assert act_of(np.zeros(1, np.float32), EPI_GELU)[0] == 0.0
    big = np.array([8.0], np.float32)
    assert act_of(big, EPI_GELU)[0] == 8.0 and act_of(-big, EPI_GELU)[0] > -1e-10


def test_relu_and_none():
    assert np.array_equal(act_of(X, EPI_RELU), np.maximum(X, 0))
    assert np.array_equal(act_of(X, EPI_NONE), X)


def test_activations_round_once_to_16_bit_outputs():
    for epi in (EPI_GELU, EPI_GELU_ERF, EPI_SIGMOID, EPI_TANH):
        y32 = act_of(X, epi, F32)
        for out in (F16, BF16):
            got = oracle.encode(out, y32)  # RNE of the fp32 value
            xb = oracle.encode(F16, X).reshape(1, -1)
            one = oracle.encode(F16, np.ones(1, np.float32)).reshape(1, 1)
            C = oracle.gemm(one, xb, 1, X.size, 1, F16, out, epi).reshape(-1)
            assert np.array_equal(C, got)


def test_nan_through_the_activations():
    nan16 = np.array([0x7e00], np.uint16).reshape(1, 1)
    one = oracle.encode(F16, np.ones(1, np.float32)).reshape(1, 1)
    for epi, want_nan in ((EPI_NONE, True), (EPI_RELU, False), (EPI_GELU, True),
                          (EPI_GELU_ERF, True), (EPI_SIGMOID, True), (EPI_TANH, True)):
        c = oracle.gemm(one, nan16, 1, 1, 1, F16, F32, epi).reshape(-1)[0]
        assert np.isnan(c) == want_nan, epi
        if not want_nan:
            assert c == 0 and not np.signbit(c)


@pytest.mark.parametrize("epi", [EPI_NONE, EPI_RELU, EPI_SIGMOID])
def test_bias_is_added_to_every_row_before_the_activation(epi):
    rng = np.random.default_rng(7)
    M = N = 24
    B = rng.integers(-4, 5, (M, N)).astype(np.float32)
    bias = rng.integers(-8, 9, N).astype(np.float32)
    I = oracle.encode(F16, np.eye(M, dtype=np.float32))
    Bb = oracle.encode(F16, B)
    C = oracle.gemm(I, Bb, M, N, M, F16, F32, epi, bias=bias).reshape(M, N)
    v = B + bias[None, :]  # exact: small integers
    want = {EPI_NONE: v, EPI_RELU: np.maximum(v, 0),
            EPI_SIGMOID: special.expit(v.astype(np.float64)).astype(np.float32)}[epi]
    assert ulps(C, want).max() <= 1


def test_bias_is_shared_by_batch_items_and_sampled_agrees():
    rng = np.random.default_rng(8)
    M, N, K, batch = 5, 7, 9, 3
    A = oracle.encode(BF16, rng.standard_normal((batch, M, K)).astype(np.float32))
    B = oracle.encode(BF16, rng.standard_normal((batch, K, N)).astype(np.float32))
    bias = rng.standard_normal(N).astype(np.float32)
    C0, Y0 = oracle.gemm(A, B, M, N, K, BF16, F32, EPI_NONE, batch=batch, want_y=True)
    C1, Y1 = oracle.gemm(A, B, M, N, K, BF16, F32, EPI_TANH, batch=batch, want_y=True, bias=bias)
    want = np.tanh((Y0 + bias[None, None, :]).astype(np.float32).astype(np.float64)).astype(np.float32)
    assert ulps(Y1, want).max() <= 1
    bi, ii, jj = np.meshgrid(np.arange(batch), np.arange(M), np.arange(N), indexing="ij")
    out, Ys = oracle.gemm_sampled(A, B, M, N, K, BF16, F32, EPI_TANH, bi.ravel(), ii.ravel(),
                                  jj.ravel(), batch=batch, bias=bias)
    assert np.array_equal(Ys, Y1.ravel())


# Wide grid for the GELU tanh form: every fp16-exact value in [-8, 8) at
# steps of 1/64, plus a log-spaced sweep of magnitudes out to 30 (fp32
# values, exact in fp16 after encoding) where x^3 dominates the argument.
def _wide_gelu_grid():
    mags = np.geomspace(1e-3, 30.0, 2001)
    wide = np.concatenate([mags, -mags]).astype(np.float32)
    wide = oracle.decode(F16, oracle.encode(F16, wide))  # exact as fp16 operands
    return np.unique(np.concatenate([X, wide]))


def test_gelu_tanh_form_matches_torch_in_double():
    # An implementation other than the oracle's: torch's GELU with
    # approximate="tanh", evaluated on float64 tensors, then rounded once to
    # fp32 as the oracle does.  The form x(1 + tanh(sqrt(2/pi)(x + c x^3)))/2
    # is the published tanh approximation of x Phi(x) (Hendrycks and Gimpel,
    # "Gaussian Error Linear Units", 2016), c = 0.044715.  A change of c in
    # its fifth digit, or of sqrt(2/pi) by 1e-3, moves many grid points by
    # tens of ulps; the bound below admits only double's own rounding.
    import torch
    xs = _wide_gelu_grid()
    got = act_of(xs, EPI_GELU)
    want = torch.nn.functional.gelu(torch.from_numpy(xs.astype(np.float64)),
                                    approximate="tanh").numpy()
    # Below -5, 1 + tanh cancels in double (both sides evaluate the same
    # form), leaving an absolute error of about 1e-16 |x| on top of the one
    # fp32 rounding: there the bound is one fp32 ulp of the result plus that.
    tail = xs < -5
    assert ulps(got[~tail], want[~tail].astype(np.float32)).max() <= 1
    w32 = want[tail].astype(np.float32)
    bound = np.spacing(np.abs(w32)).astype(np.float64) + 4e-16 * np.abs(xs[tail])
    assert np.all(np.abs(got[tail].astype(np.float64) - want[tail]) <= bound)


def test_gelu_tanh_form_constants_are_observable():
    # Guard the pin above: perturbing either constant in a double-precision
    # twin of the form moves the result by more than the 1-ulp bound on this
    # grid, so the pin could not pass with a wrong constant.
    xs = _wide_gelu_grid().astype(np.float64)
    xs = xs[xs > -5]

    def form(c, s):
        return (0.5 * xs * (1.0 + np.tanh(s * (xs + c * xs ** 3)))).astype(np.float32)

    import torch
    ref = torch.nn.functional.gelu(torch.from_numpy(xs), approximate="tanh").numpy().astype(np.float32)
    s0 = np.sqrt(2.0 / np.pi)
    assert ulps(form(0.044715, s0), ref).max() <= 1
    assert ulps(form(0.0447, s0), ref).max() > 1
    assert ulps(form(0.044715, s0 * 1.001), ref).max() > 1
