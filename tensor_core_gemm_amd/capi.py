"""ctypes binding of include/tcgemm.h: the same entry points, marshalling only.

Every computation happens in libtcgemm.so; this module converts Python
values and torch tensors (device memory, streams) into the C arguments and
turns negative return codes into GemmError.
"""
from __future__ import annotations

import ctypes
import re

import torch

from ._lib import lib

F32, F16, BF16, FP8 = 0, 4, 5, 9
EPI_NONE, EPI_RELU, EPI_GELU, EPI_GELU_ERF, EPI_SIGMOID, EPI_TANH = 0, 1, 2, 3, 4, 5
FLAG_FORCE_STAGES_1, FLAG_UNSTAGED, FLAG_FORCE_STAGES_2, FLAG_BIAS, FLAG_SPLIT_K = 1, 2, 4, 8, 16
FLAG_TUNED = 32

GEMM_OK = 0
GEMM_E_ARG, GEMM_E_DTYPE, GEMM_E_ALIGN, GEMM_E_ALIAS = -1, -2, -3, -4
GEMM_E_DEVICE, GEMM_E_LAUNCH, GEMM_E_NOMEM, GEMM_E_PLAN, GEMM_E_SIZE = -5, -6, -7, -8, -9
GEMM_E_WORKSPACE, GEMM_E_SCRATCH = -10, -11
NOALLOC_SCRATCH_BYTES = 64 << 20  # GEMM_NOALLOC_SCRATCH_BYTES

TORCH_TO_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16,
                 torch.float8_e4m3fn: FP8}
CODE_TO_TORCH = {v: k for k, v in TORCH_TO_CODE.items()}


class gemm_desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("epilogue", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("batch", ctypes.c_int64), ("stride_a", ctypes.c_int64),
                ("stride_b", ctypes.c_int64), ("stride_c", ctypes.c_int64),
                ("tile", ctypes.c_int32), ("split_k", ctypes.c_int32)]


class gemm_device_caps(ctypes.Structure):
    _fields_ = [("num_cus", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("async_copy", ctypes.c_int32), ("wave_size", ctypes.c_int32),
                ("clock_khz", ctypes.c_int32), ("num_xcds", ctypes.c_int32),
                ("arch", ctypes.c_char * 64)]


class gemm_plan_info(ctypes.Structure):
    _fields_ = [("tile_id", ctypes.c_int32), ("bm", ctypes.c_int32), ("bn", ctypes.c_int32),
                ("bk", ctypes.c_int32), ("waves", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("vec16", ctypes.c_int32),
                ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64),
                ("workgroups", ctypes.c_int64), ("trips", ctypes.c_int64),
                ("mfma_per_run", ctypes.c_int64), ("mfma_m", ctypes.c_int32),
                ("mfma_n", ctypes.c_int32), ("mfma_k", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("trips_per_split", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("tail_rows", ctypes.c_int64),
                ("tail_split", ctypes.c_int32), ("reserved0", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class gemm_run_args(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_int64), ("reserved", ctypes.c_int64 * 4)]


_vp = ctypes.c_void_p
_SIGS = {
    "gemm_device_caps_query": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(gemm_device_caps)]),
    "gemm_plan": (ctypes.c_int, [ctypes.POINTER(gemm_desc), ctypes.POINTER(_vp)]),
    "gemm_plan_for_caps": (ctypes.c_int, [ctypes.POINTER(gemm_desc),
                                          ctypes.POINTER(gemm_device_caps), ctypes.POINTER(_vp)]),
    "gemm_plan_get_info": (ctypes.c_int, [_vp, ctypes.POINTER(gemm_plan_info)]),
    "gemm_plan_describe": (ctypes.c_char_p, [_vp]),
    "gemm_run": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp]),
    "gemm_run_ex": (ctypes.c_int, [_vp, _vp, _vp, _vp, ctypes.c_void_p, _vp]),
    "gemm_run_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp]),
    "gemm_plan_destroy": (None, [_vp]),
    "gemm_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "gemm_stage_depth": (ctypes.c_int, [ctypes.POINTER(gemm_device_caps), ctypes.c_int64,
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_int]),
    "gemm_tile_count": (ctypes.c_int, []),
    "gemm_autotune": (ctypes.c_int, [ctypes.POINTER(gemm_desc), _vp, _vp, _vp, ctypes.c_void_p, _vp,
                                     ctypes.POINTER(_vp)]),
    "gemm_tune_cache_save": (ctypes.c_int, [ctypes.c_char_p]),
    "gemm_tune_cache_load": (ctypes.c_int, [ctypes.c_char_p]),
    "gemm_tune_cache_clear": (None, []),
    "gemm_tune_cache_size": (ctypes.c_int, []),
    "gemm_runtime_version": (ctypes.c_int, []),
}
_fns = {}


def _fn(name):
    f = _fns.get(name)
    if f is None:
        f = getattr(lib(), name)
        f.restype, f.argtypes = _SIGS[name]
        _fns[name] = f
    return f


class GemmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {gemm_strerror(code)} (code {code})")


def _check(code: int, where: str):
    if code != GEMM_OK:
        raise GemmError(code, where)


def gemm_strerror(code: int) -> str:
    return _fn("gemm_strerror")(code).decode()


def gemm_tile_count() -> int:
    return _fn("gemm_tile_count")()


def gemm_runtime_version() -> int:
    return _fn("gemm_runtime_version")()


def gemm_device_caps_query(device: int = 0) -> gemm_device_caps:
    caps = gemm_device_caps()
    _check(_fn("gemm_device_caps_query")(device, ctypes.byref(caps)), "gemm_device_caps_query")
    return caps


def make_caps(num_cus=256, lds_bytes=163840, async_copy=1, wave_size=64, clock_khz=2400000,
              num_xcds=8, arch=b"gfx950:sramecc+:xnack-") -> gemm_device_caps:
    """A capability record for host-only planning (no device needed)."""
    return gemm_device_caps(num_cus, lds_bytes, async_copy, wave_size, clock_khz, num_xcds, arch)


def gemm_stage_depth(caps: gemm_device_caps, used: int, tile_bytes, stage_enabled: bool = True) -> int:
    arr = (ctypes.c_int64 * max(len(tile_bytes), 1))(*tile_bytes)
    return _fn("gemm_stage_depth")(ctypes.byref(caps), used, arr, len(tile_bytes),
                                   1 if stage_enabled else 0)


def make_desc(M, N, K, in_dtype=F16, out_dtype=F32, epilogue=EPI_NONE, flags=0, batch=1,
              stride_a=0, stride_b=0, stride_c=0, tile=0, split_k=0) -> gemm_desc:
    return gemm_desc(M, N, K, in_dtype, out_dtype, epilogue, flags, batch, stride_a, stride_b,
                     stride_c, tile, split_k)


class Plan:
    """Owns a gemm_plan_t; destroyed with the object."""

    def __init__(self, handle: int, desc: gemm_desc):
        self._h = _vp(handle)
        self.desc = desc

    @property
    def handle(self):
        return self._h

    def info(self) -> gemm_plan_info:
        return gemm_plan_get_info(self)

    def describe(self) -> str:
        return gemm_plan_describe(self)

    def close(self):
        if self._h and self._h.value:
            _fn("gemm_plan_destroy")(self._h)
            self._h = _vp(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gemm_plan(desc: gemm_desc) -> Plan:
    h = _vp()
    _check(_fn("gemm_plan")(ctypes.byref(desc), ctypes.byref(h)), "gemm_plan")
    return Plan(h.value, desc)


def gemm_plan_for_caps(desc: gemm_desc, caps: gemm_device_caps) -> Plan:
    h = _vp()
    _check(_fn("gemm_plan_for_caps")(ctypes.byref(desc), ctypes.byref(caps), ctypes.byref(h)),
           "gemm_plan_for_caps")
    return Plan(h.value, desc)


def gemm_plan_get_info(plan: Plan) -> gemm_plan_info:
    info = gemm_plan_info()
    _check(_fn("gemm_plan_get_info")(plan.handle, ctypes.byref(info)), "gemm_plan_get_info")
    return info


def gemm_plan_describe(plan: Plan) -> str:
    return _fn("gemm_plan_describe")(plan.handle).decode()


def gemm_plan_destroy(plan: Plan) -> None:
    plan.close()


def _ptr(x, need: int = 0, what: str = "buffer") -> int | None:
    """The device address of a tensor or a raw pointer (an int, passed as
    is).  A tensor must be a contiguous GPU tensor of at least `need` bytes:
    a host tensor or a short one would hand the kernels an address they
    cannot read or write within bounds."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"{what} is not a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{what} is not contiguous")
    have = x.numel() * x.element_size()
    if have < need:
        raise ValueError(f"{what} holds {have} bytes; the plan needs {need}")
    return x.data_ptr()


_IN_BYTES = {F16: 2, BF16: 2, FP8: 1}
_OUT_BYTES = {F32: 4, F16: 2, BF16: 2}


def _extent(batch: int, stride: int, rows: int, cols: int) -> int:
    """Elements an operand spans: one item, or batch items `stride` apart."""
    if rows == 0 or cols == 0:
        return 0
    return rows * cols if batch <= 1 else (batch - 1) * stride + rows * cols


def _needs(desc: gemm_desc | None) -> tuple:
    """Bytes A, B, C and a bias must hold for a description (none without one:
    the library rejects a plan that has none)."""
    if desc is None:
        return 0, 0, 0, 0
    ib, ob = _IN_BYTES.get(desc.in_dtype, 2), _OUT_BYTES.get(desc.out_dtype, 4)
    b = desc.batch
    return (_extent(b, desc.stride_a, desc.M, desc.K) * ib, _extent(b, desc.stride_b, desc.K, desc.N) * ib,
            _extent(b, desc.stride_c, desc.M, desc.N) * ob, desc.N * 4)


def _operands(needs: tuple, A, B, C, bias=None):
    """Device addresses of A, B, C (and bias), tensors checked against the
    byte counts of `needs`."""
    return (_ptr(A, needs[0], "A"), _ptr(B, needs[1], "B"), _ptr(C, needs[2], "C"),
            _ptr(bias, needs[3], "bias"))


def _plan_needs(plan) -> tuple:
    """_needs of a plan's description, computed once (a plan is immutable)."""
    n = plan.__dict__.get("_needs")
    if n is None:
        n = _needs(plan.desc)
        plan._needs = n
    return n


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def gemm_run(plan: Plan, A, B, C, stream=None) -> None:
    """Launch on `stream` (a torch.cuda.Stream, a raw hipStream_t int, or
    None for torch's current stream).  A, B, C are device tensors or raw
    device pointers; nothing is synchronised."""
    a, b, c, _ = _operands(_plan_needs(plan), A, B, C)
    _check(_fn("gemm_run")(plan.handle, a, b, c, _stream(stream)), "gemm_run")


def gemm_run_ex(plan: Plan, A, B, C, bias=None, workspace=None, workspace_bytes=None,
                stream=None) -> None:
    """gemm_run with a bias (N fp32 values on the device) and a workspace
    (device memory of at least the plan's workspace_bytes, 256-byte aligned);
    tensors or raw device pointers."""
    if workspace_bytes is None:
        workspace_bytes = 0
        if workspace is not None and not isinstance(workspace, int):
            workspace_bytes = workspace.numel() * workspace.element_size()
    a, b, c, bp = _operands(_plan_needs(plan), A, B, C, bias)
    args = gemm_run_args(bp, _ptr(workspace, 0, "workspace"), workspace_bytes)
    _check(_fn("gemm_run_ex")(plan.handle, a, b, c, ctypes.byref(args), _stream(stream)),
           "gemm_run_ex")


def gemm_run_noalloc(plan: Plan, A, B, C, bias=None, stream=None) -> None:
    """gemm_run_ex with the library's fixed device array as the split-K
    workspace (no device allocation; calls that overlap on one GPU race)."""
    a, b, c, bp = _operands(_plan_needs(plan), A, B, C, bias)
    _check(_fn("gemm_run_noalloc")(plan.handle, a, b, c, bp, _stream(stream)), "gemm_run_noalloc")


def check_runtime() -> None:
    """The library must run on the HIP runtime torch loaded (one per process)."""
    v = gemm_runtime_version()
    hip = torch.version.hip
    if hip:
        m = re.match(r"(\d+)\.(\d+)\.(\d+)", hip)
        if m:
            want = int(m.group(1)) * 10_000_000 + int(m.group(2)) * 100_000 + int(m.group(3))
            if v != want:
                raise RuntimeError(f"libtcgemm.so runs on HIP runtime {v}, torch on {want}: "
                                   "two HIP runtimes are loaded")


def gemm_autotune(desc: gemm_desc, A, B, C, bias=None, workspace=None, workspace_bytes=None,
                  stream=None) -> Plan:
    """Time the candidate configurations on these buffers, keep the fastest
    in the library's cache and return its plan (synchronises the stream)."""
    if workspace_bytes is None:
        workspace_bytes = 0
        if workspace is not None and not isinstance(workspace, int):
            workspace_bytes = workspace.numel() * workspace.element_size()
    a, b, c, bp = _operands(_needs(desc), A, B, C, bias)
    args = gemm_run_args(bp, _ptr(workspace, 0, "workspace"), workspace_bytes)
    h = _vp()
    _check(_fn("gemm_autotune")(ctypes.byref(desc), a, b, c, ctypes.byref(args),
                                _stream(stream), ctypes.byref(h)), "gemm_autotune")
    return Plan(h.value, desc)


def gemm_tune_cache_save(path: str) -> None:
    _check(_fn("gemm_tune_cache_save")(path.encode()), "gemm_tune_cache_save")


def gemm_tune_cache_load(path: str) -> None:
    _check(_fn("gemm_tune_cache_load")(path.encode()), "gemm_tune_cache_load")


def gemm_tune_cache_clear() -> None:
    _fn("gemm_tune_cache_clear")()


def gemm_tune_cache_size() -> int:
    return _fn("gemm_tune_cache_size")()
