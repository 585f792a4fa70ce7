"""tensor_core_gemm_amd -- C = epilogue(A . B) on AMD Instinct MI355X (gfx950).

The computation lives in libtcgemm.so (hand-written HIP kernels behind the C
ABI of include/tcgemm.h).  This package binds that ABI with ctypes under the
same names (gemm_plan, gemm_run, ...) and adds ``matmul`` for torch tensors.
torch serves only for device memory and streams.  If the library is not
built, importing the package fails: there is no fallback path.
"""
from __future__ import annotations

import torch

from .capi import (BF16, EPI_NONE, EPI_RELU, F16, F32, FLAG_FORCE_STAGES_1, FLAG_FORCE_STAGES_2,
                   FLAG_UNSTAGED,
                   GEMM_E_ALIAS, GEMM_E_ALIGN, GEMM_E_ARG, GEMM_E_DEVICE, GEMM_E_DTYPE,
                   GEMM_E_LAUNCH, GEMM_E_NOMEM, GEMM_E_PLAN, GEMM_E_SIZE, GEMM_OK, CODE_TO_TORCH,
                   TORCH_TO_CODE, GemmError, Plan, check_runtime, gemm_desc, gemm_device_caps,
                   gemm_device_caps_query, gemm_plan, gemm_plan_describe, gemm_plan_destroy,
                   gemm_plan_for_caps, gemm_plan_get_info, gemm_plan_info, gemm_run,
                   gemm_runtime_version, gemm_stage_depth, gemm_strerror, gemm_tile_count,
                   make_caps, make_desc)
from ._lib import LIB_PATH, lib

lib()  # fail loudly now if the library is missing

_plan_cache: dict = {}


def plan_for(M, N, K, in_dtype, out_dtype, epilogue=EPI_NONE, flags=0, batch=1, stride_a=0,
             stride_b=0, stride_c=0, tile=0) -> Plan:
    """A cached plan for the current device (plans are immutable)."""
    key = (torch.cuda.current_device(), M, N, K, in_dtype, out_dtype, epilogue, flags, batch,
           stride_a, stride_b, stride_c, tile)
    p = _plan_cache.get(key)
    if p is None:
        p = gemm_plan(make_desc(M, N, K, in_dtype, out_dtype, epilogue, flags, batch, stride_a,
                                stride_b, stride_c, tile))
        _plan_cache[key] = p
    return p


def matmul(A: torch.Tensor, B: torch.Tensor, *, relu: bool = False, out_dtype=None,
           out: torch.Tensor | None = None, flags: int = 0, tile: int = 0,
           stream=None) -> torch.Tensor:
    """C = relu?(A @ B) with fp32 accumulation on the MFMA units.

    A is [M, K] or [batch, M, K], B is [K, N] or [batch, K, N]; both fp16 or
    both bf16, row-major and contiguous, on the GPU.  out_dtype is
    torch.float32, float16 or bfloat16 (default: the input type).
    """
    if A.dtype not in (torch.float16, torch.bfloat16) or B.dtype != A.dtype:
        raise TypeError("A and B must share one dtype, float16 or bfloat16")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("A and B must be on the same GPU")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous (row-major)")
    if A.dim() != B.dim() or A.dim() not in (2, 3):
        raise ValueError("A and B must both be 2-d or both 3-d")
    batch = A.shape[0] if A.dim() == 3 else 1
    if A.dim() == 3 and B.shape[0] != batch:
        raise ValueError("batch sizes differ")
    M, K = A.shape[-2], A.shape[-1]
    K2, N = B.shape[-2], B.shape[-1]
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    odt = out_dtype or A.dtype
    if odt not in TORCH_TO_CODE:
        raise TypeError("out_dtype must be float32, float16 or bfloat16")
    shape = (batch, M, N) if A.dim() == 3 else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=odt, device=A.device)
    elif tuple(out.shape) != shape or out.dtype != odt or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    with torch.cuda.device(A.device):
        p = plan_for(M, N, K, TORCH_TO_CODE[A.dtype], TORCH_TO_CODE[odt],
                     EPI_RELU if relu else EPI_NONE, flags, batch,
                     M * K if batch > 1 else 0, K * N if batch > 1 else 0,
                     M * N if batch > 1 else 0, tile)
        gemm_run(p, A, B, out, stream)
    return out


__all__ = [n for n in dir() if not n.startswith("_")]
