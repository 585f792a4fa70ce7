"""Bindings for the layout probes declared in include/tcgemm_probe.h."""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import lib

MFMA_32x32x16_BF16, MFMA_32x32x16_F16, MFMA_16x16x32_BF16, MFMA_16x16x32_F16 = 0, 1, 2, 3
MFMA_32x32x64_FP8 = 4  # register-only rate probe only

_vp = ctypes.c_void_p


def _fn(name, argtypes):
    f = getattr(lib(), name)
    f.argtypes = argtypes
    f.restype = ctypes.c_int
    return f


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def mfma(kind: int, a_regs: np.ndarray, b_regs: np.ndarray) -> np.ndarray:
    """Run one MFMA: a_regs/b_regs are [64, 8] uint16 per-lane register
    contents; returns the [64, 16] float32 result registers."""
    a = torch.from_numpy(np.ascontiguousarray(a_regs, np.uint16).view(np.int16)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(b_regs, np.uint16).view(np.int16)).cuda()
    d = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    f = _fn("tcg_probe_mfma", [ctypes.c_int, _vp, _vp, _vp, _vp])
    _check(f(kind, a.data_ptr(), b.data_ptr(), d.data_ptr(), _stream()), "tcg_probe_mfma")
    torch.cuda.synchronize()
    return d.cpu().numpy().reshape(64, 16)


def ds_read_tr16(lds_init: np.ndarray, lane_byte_addr: np.ndarray) -> np.ndarray:
    init = torch.from_numpy(np.ascontiguousarray(lds_init, np.uint16).view(np.int16)).cuda()
    addr = np.ascontiguousarray(lane_byte_addr, np.uint32)
    assert addr.shape == (64,)
    out = torch.zeros(64 * 4, dtype=torch.int16, device="cuda")
    f = _fn("tcg_probe_ds_read_tr16", [_vp, ctypes.c_int, _vp, _vp, _vp])
    _check(f(init.data_ptr(), init.numel(), addr.ctypes.data_as(_vp), out.data_ptr(), _stream()),
           "tcg_probe_ds_read_tr16")
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16).reshape(64, 4)


def buffer_lds(src: torch.Tensor, num_records: int, lane_voffset: np.ndarray,
               lds_byte_base: int) -> np.ndarray:
    voff = np.ascontiguousarray(lane_voffset, np.uint32)
    assert voff.shape == (64,) and src.is_cuda and src.dtype == torch.int32
    out = torch.zeros(2048, dtype=torch.int32, device="cuda")
    f = _fn("tcg_probe_buffer_lds", [_vp, ctypes.c_uint32, _vp, ctypes.c_uint32, _vp, _vp])
    _check(f(src.data_ptr(), num_records, voff.ctypes.data_as(_vp), lds_byte_base,
             out.data_ptr(), _stream()), "tcg_probe_buffer_lds")
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def mfma_f8(a_regs: np.ndarray, b_regs: np.ndarray) -> np.ndarray:
    """One FP8 E4M3 32x32x64 MFMA: a_regs/b_regs are [64, 32] uint8 per-lane
    register bytes; returns the [64, 16] float32 result registers."""
    a = torch.from_numpy(np.ascontiguousarray(a_regs, np.uint8)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(b_regs, np.uint8)).cuda()
    d = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    f = _fn("tcg_probe_mfma_f8", [_vp, _vp, _vp, _vp])
    _check(f(a.data_ptr(), b.data_ptr(), d.data_ptr(), _stream()), "tcg_probe_mfma_f8")
    torch.cuda.synchronize()
    return d.cpu().numpy().reshape(64, 16)


def ds_read_tr8(lds_init: np.ndarray, lane_byte_addr: np.ndarray) -> np.ndarray:
    init = torch.from_numpy(np.ascontiguousarray(lds_init, np.uint8)).cuda()
    addr = np.ascontiguousarray(lane_byte_addr, np.uint32)
    assert addr.shape == (64,)
    out = torch.zeros(64 * 8, dtype=torch.uint8, device="cuda")
    f = _fn("tcg_probe_ds_read_tr8", [_vp, ctypes.c_int, _vp, _vp, _vp])
    _check(f(init.data_ptr(), init.numel(), addr.ctypes.data_as(_vp), out.data_ptr(), _stream()),
           "tcg_probe_ds_read_tr8")
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(64, 8)


# ---------------------------------------------------------------------------
# Measurement probes: the shader clock and the register-only MFMA rate.

def wallclock_khz(device: int = 0) -> int:
    """Rate of the constant clock that s_memrealtime counts, in kHz."""
    v = ctypes.c_int(0)
    f = _fn("tcg_probe_wallclock_khz", [ctypes.c_int, ctypes.POINTER(ctypes.c_int)])
    _check(f(device, ctypes.byref(v)), "tcg_probe_wallclock_khz")
    return int(v.value)


class ClockProbe:
    """Average shader clock per XCD between two marks on one stream.

    Each mark launches `workgroups` one-wave workgroups that record the XCD
    they run on, the shader-clock counter and the constant-rate counter;
    per XCD, the clock between the marks is the difference of the first
    counter's medians over the difference of the second's, times the
    constant rate."""

    def __init__(self, workgroups: int = 2048, device: int = 0):
        self.wg = workgroups
        self.bufs = [torch.zeros(3 * workgroups, dtype=torch.int64, device="cuda") for _ in range(2)]
        self.khz = wallclock_khz(device)
        self._f = _fn("tcg_probe_clock", [ctypes.c_int, _vp, _vp])

    def mark(self, which: int, stream=None):
        s = ctypes.c_void_p(stream.cuda_stream if stream is not None
                            else torch.cuda.current_stream().cuda_stream)
        _check(self._f(self.wg, self.bufs[which].data_ptr(), s), "tcg_probe_clock")

    def result(self) -> dict:
        """{'per_xcd_mhz': {xcd: MHz}, 'mean_mhz', 'min_mhz', 'max_mhz',
        'seconds'} (call after both marks and a synchronisation)."""
        a = self.bufs[0].cpu().numpy().reshape(-1, 3)
        b = self.bufs[1].cpu().numpy().reshape(-1, 3)
        per = {}
        span = []
        for x in sorted(set(a[:, 0].tolist()) & set(b[:, 0].tolist())):
            ta, ra = a[a[:, 0] == x, 1], a[a[:, 0] == x, 2]
            tb, rb = b[b[:, 0] == x, 1], b[b[:, 0] == x, 2]
            dt = float(np.median(tb)) - float(np.median(ta))
            dr = float(np.median(rb)) - float(np.median(ra))
            if dr > 0:
                per[int(x)] = round(dt / dr * self.khz / 1e3, 1)
                span.append(dr / (self.khz * 1e3))
        vals = list(per.values())
        return {"per_xcd_mhz": per,
                "mean_mhz": round(float(np.mean(vals)), 1) if vals else None,
                "min_mhz": min(vals) if vals else None,
                "max_mhz": max(vals) if vals else None,
                "seconds": round(float(np.mean(span)), 6) if span else None}


def mfma_rate(kind: int, workgroups: int, iters: int, operands: torch.Tensor, sink: torch.Tensor,
              ticks: torch.Tensor, stream=None):
    """One launch of the register-only MFMA loop (tcg_probe_mfma_rate):
    operands is a device tensor of 16 * 64 * 16 bytes (16-bit kinds: 8
    values per lane and register set) or 16 * 64 * 32 bytes (FP8), sink a
    float32 tensor of workgroups * 256, ticks an int64 tensor of
    workgroups.  Returns the flops the launch performs."""
    need = 16 * 64 * (32 if kind == MFMA_32x32x64_FP8 else 16)
    assert operands.is_cuda and operands.numel() * operands.element_size() >= need
    assert sink.numel() >= workgroups * 256 and ticks.numel() >= workgroups
    s = ctypes.c_void_p(stream.cuda_stream if stream is not None
                        else torch.cuda.current_stream().cuda_stream)
    f = _fn("tcg_probe_mfma_rate", [ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp])
    _check(f(kind, workgroups, iters, operands.data_ptr(), sink.data_ptr(), ticks.data_ptr(), s),
           "tcg_probe_mfma_rate")
    per_mfma = {MFMA_32x32x16_BF16: 32768, MFMA_32x32x16_F16: 32768,
                MFMA_32x32x64_FP8: 131072}.get(kind, 16384)
    return workgroups * 4 * iters * 64 * per_mfma


# pattern: (name, waves per workgroup, MFMAs per round per wave)
COPY_PATTERNS = {0: ("4 waves, no copies", 4, 32), 1: ("4 waves, 8 copies, 1 per 4 MFMAs", 4, 32),
                 2: ("4 waves, 8 copies, 2 bursts of 4", 4, 32), 3: ("8 waves, no copies", 8, 32),
                 4: ("8 waves, 4 copies each (same per SIMD as 1)", 8, 32),
                 5: ("8 waves, 8 copies each (twice 1 per SIMD)", 8, 32),
                 6: ("4 waves, no copies, 16x16x32 MFMAs", 4, 64),
                 7: ("4 waves, 8 copies, 1 per 8 16x16x32 MFMAs (same per flop as 1)", 4, 64)}
# flops of one MFMA of each pattern's shape
COPY_PATTERN_MFMA_FLOPS = {p: (16384 if rm == 64 else 32768) for p, (_, _, rm) in COPY_PATTERNS.items()}


def copy_issue(pattern: int, workgroups: int, iters: int, operands: torch.Tensor, src: torch.Tensor,
               sink: torch.Tensor, ticks: torch.Tensor, stream=None):
    """One launch of tcg_probe_copy_issue; returns the MFMAs one SIMD issues
    (for cycles per MFMA per SIMD = ticks / that)."""
    assert operands.is_cuda and operands.numel() * operands.element_size() >= 8 * 64 * 8 * 2
    assert src.is_cuda and src.numel() * src.element_size() >= 65536
    assert sink.numel() >= workgroups * 512 and ticks.numel() >= workgroups
    s = ctypes.c_void_p(stream.cuda_stream if stream is not None
                        else torch.cuda.current_stream().cuda_stream)
    f = _fn("tcg_probe_copy_issue", [ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp, _vp])
    _check(f(pattern, workgroups, iters, operands.data_ptr(), src.data_ptr(), sink.data_ptr(),
             ticks.data_ptr(), s), "tcg_probe_copy_issue")
    _, waves, per_round = COPY_PATTERNS[pattern]
    return iters * per_round * (waves // 4)
