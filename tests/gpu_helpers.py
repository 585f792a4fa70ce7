"""Shared helpers for the GPU parity tests: run the HIP path through the C
ABI and compare with the oracle."""
import sys

import numpy as np
import torch

import gemm_workloads as gw
import oracle

TOL = 1e-2  # max relative error on non-integer inputs (fp16/bf16 in, fp32 accumulate)


def note(msg):
    """Name the case before a GPU step (so a crash log says what ran)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def out_torch(dtype):
    return gw.TORCH_DTYPE[dtype]


def run(tcg, A, B, w, flags=0, tile=0, guard=0, sentinel=None, plan=None, a_offset=0,
        b_offset=0, bias=None, split_k=0, ws_fill=None):
    """Run C = epilogue(A.B + bias) on the GPU; A, B (and bias) are CPU
    tensors.  With guard > 0 the output sits inside a larger buffer filled
    with `sentinel` bits; returns (C, whole buffer, plan) on the CPU.
    a_offset/b_offset shift the operands by that many elements inside their
    device buffers.  A split-K plan gets a workspace filled with ws_fill
    (NaN by default: its contents on entry must not matter)."""
    dev = torch.device("cuda")
    Ad = torch.empty(A.numel() + a_offset, dtype=A.dtype, device=dev)
    Ad[a_offset:].copy_(A.reshape(-1))
    Bd = torch.empty(B.numel() + b_offset, dtype=B.dtype, device=dev)
    Bd[b_offset:].copy_(B.reshape(-1))
    n_out = w.batch * w.M * w.N
    odt = out_torch(w.out_dtype)
    buf = torch.empty(n_out + 2 * guard, dtype=odt, device=dev)
    if sentinel is not None:
        buf.view(torch.int32 if odt == torch.float32 else torch.int16).fill_(sentinel)
    else:
        buf.zero_()
    C = buf[guard:guard + n_out]
    if bias is not None:
        flags |= tcg.FLAG_BIAS
    if plan is None:
        plan = tcg.gemm_plan(tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                                           flags, w.batch,
                                           w.M * w.K if w.batch > 1 else 0,
                                           w.K * w.N if w.batch > 1 else 0,
                                           w.M * w.N if w.batch > 1 else 0, tile, split_k))
    note(f"{w.name} M={w.M} N={w.N} K={w.K} batch={w.batch} epi={w.epilogue} flags={flags} "
         f"tile={tile} split_k={split_k} plan: {plan.describe()}")
    ws_bytes = plan.info().workspace_bytes
    ws = None
    if ws_bytes:
        ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=dev)
        ws.fill_(float("nan") if ws_fill is None else ws_fill)
    bias_d = bias.to(dev, torch.float32).contiguous() if bias is not None else None
    a_arg = Ad[a_offset:] if a_offset else Ad
    b_arg = Bd[b_offset:] if b_offset else Bd
    if bias_d is None and ws is None:
        tcg.gemm_run(plan, a_arg, b_arg, C)
    else:
        tcg.gemm_run_ex(plan, a_arg, b_arg, C, bias=bias_d, workspace=ws)
    torch.cuda.synchronize()
    shape = (w.batch, w.M, w.N)
    return C.cpu().reshape(shape), buf.cpu(), plan


def as_bits(C):
    """Output tensor -> numpy array of raw bits (for bitwise comparisons)."""
    t = C.contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.view(torch.int16).numpy()


def as_values(C):
    return C.float().numpy()


def rel_errors(c, y, sigma):
    """|c - y| / max(|y|, 0.01 sigma): relative error with a floor at one
    hundredth of an output's standard deviation (half of the relu outputs
    are 0, where a plain relative error is undefined)."""
    c = np.asarray(c, np.float64)
    y = np.asarray(y, np.float64)
    return np.abs(c - y) / np.maximum(np.abs(y), 0.01 * sigma)


BOUNDED = (4, 5)  # sigmoid, tanh: outputs of size <= 1


def floor_scale(w):
    """The relative-error floor's scale: the standard deviation s of an
    output before the epilogue.  For the activations whose outputs are
    bounded by 1 it is capped at 1 (a stricter floor) where the operands are
    16-bit: their MFMA sums as accurately as the oracle's fp32 fold.  The FP8
    MFMA adds each group of 8 products aligned to the group's largest and
    drops what lies more than 13 bits below it (test_gpu_fp8.py pins this),
    so its sums differ from the fp32 fold by about 1e-4 s whatever the
    activation; a bounded activation passes that on with slope at most 1, so
    FP8 keeps the uncapped floor."""
    s = w.sigma_out()
    return min(s, 1.0) if w.epilogue in BOUNDED and w.in_dtype != gw.FP8 else s


def check_against_oracle(w, A, B, C, bias=None):
    """Full comparison: exact for integer workloads, TOL otherwise."""
    Cref, Y = oracle.gemm(A, B, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                          batch=w.batch, want_y=True, bias=bias)
    got = as_values(C)
    if w.exact:
        want = oracle.to_float(w.out_dtype, Cref)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{w.name}: {len(bad)} mismatches, first at {bad[:5].tolist()}"
        return 0.0
    assert np.all(np.isfinite(got)), f"{w.name}: non-finite output"
    err = rel_errors(got, Y, floor_scale(w))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL, f"{w.name}: max rel err {worst:.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    return worst


def check_sampled(w, A, B, C, count=4096, seed=123, bias=None):
    bi, ii, jj = gw.sample_indices(w.M, w.N, count, seed, w.batch)
    out, Y = oracle.gemm_sampled(A, B, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, bi, ii,
                                 jj, batch=w.batch, bias=bias)
    got = as_values(C)[bi, ii, jj]
    if w.exact:
        assert np.array_equal(got, oracle.to_float(w.out_dtype, out))
        return 0.0
    err = rel_errors(got, Y, floor_scale(w))
    worst = float(err.max())
    assert worst <= TOL, f"{w.name}: sampled max rel err {worst:.3e}"
    return worst
