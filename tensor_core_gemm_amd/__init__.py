"""tensor_core_gemm_amd -- C = epilogue(A . B) on AMD Instinct MI355X (gfx950).

The computation lives in libtcgemm.so (hand-written HIP kernels behind the C
ABI of include/tcgemm.h).  This package binds that ABI with ctypes under the
same names (gemm_plan, gemm_run, ...) and adds ``matmul`` for torch tensors.
torch serves only for device memory and streams.  If the library is not
built, importing the package fails: there is no fallback path.
"""
from __future__ import annotations

import torch

from .capi import (BF16, FP8, EPI_GELU, EPI_GELU_ERF, EPI_NONE, EPI_RELU, EPI_SIGMOID, EPI_TANH, F16,
                   F32, FLAG_BIAS, FLAG_FORCE_STAGES_1, FLAG_FORCE_STAGES_2, FLAG_SPLIT_K,
                   FLAG_TUNED, FLAG_UNSTAGED, gemm_autotune, gemm_tune_cache_clear,
                   gemm_tune_cache_load, gemm_tune_cache_save, gemm_tune_cache_size, GEMM_E_ALIAS, GEMM_E_ALIGN, GEMM_E_ARG, GEMM_E_DEVICE,
                   GEMM_E_DTYPE, GEMM_E_LAUNCH, GEMM_E_NOMEM, GEMM_E_PLAN, GEMM_E_SIZE,
                   GEMM_E_WORKSPACE, GEMM_E_SCRATCH, NOALLOC_SCRATCH_BYTES, GEMM_OK, CODE_TO_TORCH, TORCH_TO_CODE, GemmError, Plan,
                   check_runtime, gemm_desc, gemm_device_caps, gemm_device_caps_query, gemm_plan,
                   gemm_plan_describe, gemm_plan_destroy, gemm_plan_for_caps, gemm_plan_get_info,
                   gemm_plan_info, gemm_run, gemm_run_args, gemm_run_ex, gemm_run_noalloc, gemm_runtime_version,
                   gemm_stage_depth, gemm_strerror, gemm_tile_count, make_caps, make_desc)
from ._lib import LIB_PATH, lib

lib()  # fail loudly now if the library is missing

_plan_cache: dict = {}


def plan_for(M, N, K, in_dtype, out_dtype, epilogue=EPI_NONE, flags=0, batch=1, stride_a=0,
             stride_b=0, stride_c=0, tile=0, split_k=0) -> Plan:
    """A cached plan for the current device (plans are immutable)."""
    key = (torch.cuda.current_device(), M, N, K, in_dtype, out_dtype, epilogue, flags, batch,
           stride_a, stride_b, stride_c, tile, split_k)
    p = _plan_cache.get(key)
    if p is None:
        p = gemm_plan(make_desc(M, N, K, in_dtype, out_dtype, epilogue, flags, batch, stride_a,
                                stride_b, stride_c, tile, split_k))
        _plan_cache[key] = p
    return p


_ACT = {None: EPI_NONE, "none": EPI_NONE, "relu": EPI_RELU, "gelu": EPI_GELU,
        "gelu_erf": EPI_GELU_ERF, "sigmoid": EPI_SIGMOID, "tanh": EPI_TANH}


# Workspace offered to gemm_autotune for split candidates: up to 16 ranges of
# C in fp32, at most this many bytes.
TUNE_WORKSPACE_CAP = 1 << 30


def matmul(A: torch.Tensor, B: torch.Tensor, *, relu: bool = False, act: str | None = None,
           bias: torch.Tensor | None = None, out_dtype=None, out: torch.Tensor | None = None,
           flags: int = 0, tile: int = 0, split_k: int = 0, tune: bool = False,
           stream=None) -> torch.Tensor:
    """C = act(A @ B + bias) with fp32 accumulation on the MFMA units.

    A is [M, K] or [batch, M, K], B is [K, N] or [batch, K, N]; both fp16,
    both bf16 or both float8_e4m3fn, row-major and contiguous, on the GPU.  bias is an fp32 vector
    of N values (one per column, shared by every row and batch item).  act is
    None, "relu", "gelu" (tanh form), "gelu_erf", "sigmoid" or "tanh"
    (relu=True means act="relu").  out_dtype is torch.float32, float16 or
    bfloat16 (default: the input type, bfloat16 for FP8 inputs).  The planner
    may split K into ranges where its time model says that pays (deep K, few
    output tiles; the workspace comes from torch's allocator); split_k = 1
    forbids it, split_k > 1 asks for that many ranges.  On a raw stream
    handle the planner does not split unless split_k asks for it.
    tune=True measures the configurations (split ones too) the first time a
    problem is seen and keeps the fastest (gemm_autotune); the run that
    tunes writes `out` several times.
    """
    if A.dtype not in (torch.float16, torch.bfloat16, torch.float8_e4m3fn) or B.dtype != A.dtype:
        raise TypeError("A and B must share one dtype, float16, bfloat16 or float8_e4m3fn")
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
    odt = out_dtype or (torch.bfloat16 if A.dtype == torch.float8_e4m3fn else A.dtype)
    if odt not in (torch.float32, torch.float16, torch.bfloat16):
        raise TypeError("out_dtype must be float32, float16 or bfloat16")
    if act not in _ACT:
        raise ValueError(f"unknown activation {act!r}")
    epi = EPI_RELU if relu and act is None else _ACT[act]
    if relu and act not in (None, "relu"):
        raise ValueError("relu=True conflicts with act")
    if bias is not None:
        if bias.dtype != torch.float32 or bias.numel() != N or not bias.is_contiguous() \
                or bias.device != A.device:
            raise ValueError("bias must be a contiguous float32 vector of N values on A's device")
        flags |= FLAG_BIAS
    shape = (batch, M, N) if A.dim() == 3 else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=odt, device=A.device)
    elif tuple(out.shape) != shape or out.dtype != odt or not out.is_contiguous() \
            or out.device != A.device:
        raise ValueError("out has the wrong shape, dtype, layout or device")
    if split_k == 0 and not isinstance(stream, int):
        flags |= FLAG_SPLIT_K
    with torch.cuda.device(A.device):
        strides = (M * K if batch > 1 else 0, K * N if batch > 1 else 0, M * N if batch > 1 else 0)
        if tune and not tile and not split_k:
            key = ("tuned", torch.cuda.current_device(), M, N, K, A.dtype, odt, epi, flags, batch)
            p = _plan_cache.get(key)
            if p is None:
                # Split candidates only where this run may split (not on a
                # raw stream handle, where no workspace can be kept alive),
                # so the tuner never keeps a plan the run below would refuse.
                may_split = bool(flags & FLAG_SPLIT_K)
                ws = None
                if may_split:
                    wsb = min(16 * batch * M * N * 4, TUNE_WORKSPACE_CAP)  # sums of up to 16 ranges
                    ws = torch.empty(wsb, dtype=torch.uint8, device=A.device)
                p = gemm_autotune(make_desc(M, N, K, TORCH_TO_CODE[A.dtype], TORCH_TO_CODE[odt], epi,
                                            flags, batch, *strides),
                                  A, B, out, bias=bias, workspace=ws, stream=stream)
                if ws is not None and stream is not None and not isinstance(stream, int):
                    ws.record_stream(stream)
                _plan_cache[key] = p
        else:
            p = plan_for(M, N, K, TORCH_TO_CODE[A.dtype], TORCH_TO_CODE[odt], epi, flags, batch,
                         *strides, tile, split_k)
        ws_bytes = p.info().workspace_bytes
        if ws_bytes and isinstance(stream, int):
            # torch cannot keep a temporary workspace alive for a raw stream
            raise ValueError("a split-K run on a raw stream needs gemm_run_ex with a workspace")
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=A.device) if ws_bytes else None
        gemm_run_ex(p, A, B, out, bias=bias, workspace=ws, stream=stream)
        if ws is not None and stream is not None:
            # the workspace was allocated for torch's current stream
            ws.record_stream(stream)
    return out


__all__ = [n for n in dir() if not n.startswith("_")]
