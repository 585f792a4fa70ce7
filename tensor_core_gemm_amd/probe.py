"""Bindings for the layout probes declared in include/tcgemm_probe.h."""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import lib

MFMA_32x32x16_BF16, MFMA_32x32x16_F16, MFMA_16x16x32_BF16, MFMA_16x16x32_F16 = 0, 1, 2, 3

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
