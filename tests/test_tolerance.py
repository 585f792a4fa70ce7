"""The parity tolerance against the oracle's own rounding, on the CPU.

The GPU results are compared with the oracle's fp32 fold within
1e-2 max(|y|, 0.01 s L) (s an output's standard deviation before the
epilogue, L the activation's largest slope).  The floor has to admit what
the oracle's own fold leaves in the value before the epilogue, passed
through the activation: this output of a random split problem (fp16,
516 x 165 x 1958, a bias, tanh) cancels to about 0.0103 against s = 44,
and there the oracle's fold is 1.3e-4 away from the exact sum.  That is
within the floor carried through tanh's slope, and beyond the floor
0.01 min(s, 1) that the sigmoid and tanh outputs once had.
"""
import numpy as np

import gemm_workloads as gw
import oracle
from gemm_workloads import EPI_TANH, F16
from gpu_helpers import TOL, floor_scale


def test_floor_admits_the_oracles_own_fold_error_near_a_tanh_zero():
    w = gw.custom(516, 165, 1958, F16, F16, EPI_TANH, gw.NORMAL, seed=5471)
    A, B = gw.make_inputs(w)
    b = gw.draw_bias(w.N, gw.NORMAL, seed=6471)
    r, c = 268, 88
    _, Y = oracle.gemm_sampled(A, B, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                               [0], [r], [c], bias=b)
    y = float(Y[0])
    v = float(np.dot(A[r].double().numpy(), B[:, c].double().numpy())) + float(b[c])
    fold_error = abs(np.tanh(v) - y)
    assert abs(v) < 0.02 and w.sigma_out() > 40  # a cancellation: tanh near its linear part
    assert fold_error <= TOL * max(abs(y), 0.01 * floor_scale(w))
    assert fold_error > TOL * max(abs(y), 0.01 * min(w.sigma_out(), 1.0))
