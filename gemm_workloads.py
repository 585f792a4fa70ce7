"""Seeded synthetic inputs for C = epilogue(A . B), shared by the HIP path's
tests and benchmark and by the CPU oracle.

This module holds no arithmetic of the product itself: it only draws
operands (fp32 on the CPU from a seeded ``torch.Generator``, then rounded to
fp16/bf16 by torch's ``.to``) and lists the workloads.  Both sides consume
the same 16-bit tensors, so input rounding is not part of any comparison.

Storage codes are those of the page "gizml:tile" (Constants): F32 = 0,
F16 = 4, BF16 = 5, FP8 = 9 (E4M3 operands: torch's float8_e4m3fn, the OCP
format).

The workloads (the first five are the method's configurations; the sixth
is the FP8 operand path at the headline's size):

* ``int_fp16_256``   -- fp16 256^3, integer entries in [-4, 4] (inclusive),
  relu, fp32 out.  Every partial sum is an integer below 2^24, so the fp32
  result is exact in any order: one correct answer.
* ``bf16_4096_relu`` -- bf16 4096^3, N(0, 1), relu, bf16 out.
* ``swin_proj_fp16`` -- the token projection of a 96-channel Swin layer over
  a 3840x2160 frame cut into 8x8 patches (page "d4r ... rrswin_enc2_epilogues":
  the frame size and channel count only): M = 129600 tokens, K = 96,
  N = 288 (3 x 96), A ~ N(0, 1), B ~ N(0, std 1/sqrt(96)), no epilogue,
  fp16 out.  There are no trained weights; Gaussian B stands in for them.
* ``ragged_fp16_1000`` -- fp16 1000^3, U(-1, 1), relu, fp32 out: no side is
  a tile multiple.
* ``deepk_bf16_2048x16384`` -- bf16 M = N = 2048, K = 16384, N(0, 1), no
  epilogue, bf16 out.
* ``fp8_4096_relu`` -- FP8 E4M3 4096^3, N(0, 1) rounded to E4M3, relu, bf16
  out.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

F32, F16, BF16, FP8 = 0, 4, 5, 9
EPI_NONE, EPI_RELU, EPI_GELU, EPI_GELU_ERF, EPI_SIGMOID, EPI_TANH = 0, 1, 2, 3, 4, 5

TORCH_DTYPE = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16,
               FP8: torch.float8_e4m3fn}
DTYPE_NAME = {F32: "f32", F16: "f16", BF16: "bf16", FP8: "fp8e4m3"}


@dataclass(frozen=True)
class Dist:
    """How one operand's entries are drawn before the cast to 16 bits."""
    kind: str            # "normal" | "randint" | "uniform"
    a: float = 0.0       # normal: mean; randint: low (inclusive); uniform: low
    b: float = 1.0       # normal: std;  randint: high (inclusive); uniform: high


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    in_dtype: int
    out_dtype: int
    epilogue: int
    seed: int
    dist_a: Dist
    dist_b: Dist
    batch: int = 1
    exact: bool = False            # integer inputs whose fp32 result is exact
    note: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    @property
    def algorithmic_bytes(self) -> int:
        """A and B read once, C written once."""
        in_size = 1 if self.in_dtype == FP8 else 2
        out_size = 4 if self.out_dtype == F32 else 2
        return self.batch * (in_size * (self.M * self.K + self.K * self.N) + out_size * self.M * self.N)

    def sigma_out(self) -> float:
        """Standard deviation of one output before the epilogue: sqrt(K) sA sB."""
        return math.sqrt(max(self.K, 1)) * _std(self.dist_a) * _std(self.dist_b)


def _std(d: Dist) -> float:
    if d.kind == "normal":
        return d.b
    if d.kind == "uniform":
        return (d.b - d.a) / math.sqrt(12.0)
    n = int(d.b - d.a + 1)
    return math.sqrt((n * n - 1) / 12.0)


NORMAL = Dist("normal", 0.0, 1.0)
INT4 = Dist("randint", -4, 4)
UNIT = Dist("uniform", -1.0, 1.0)

WORKLOADS = {
    w.name: w
    for w in [
        Workload("int_fp16_256", 256, 256, 256, F16, F32, EPI_RELU, 1, INT4, INT4, exact=True),
        Workload("bf16_4096_relu", 4096, 4096, 4096, BF16, BF16, EPI_RELU, 2, NORMAL, NORMAL),
        Workload("swin_proj_fp16", 129600, 288, 96, F16, F16, EPI_NONE, 3, NORMAL,
                 Dist("normal", 0.0, 1.0 / math.sqrt(96.0))),
        Workload("ragged_fp16_1000", 1000, 1000, 1000, F16, F32, EPI_RELU, 4, UNIT, UNIT),
        Workload("deepk_bf16_2048x16384", 2048, 2048, 16384, BF16, BF16, EPI_NONE, 5, NORMAL,
                 NORMAL),
        Workload("fp8_4096_relu", 4096, 4096, 4096, FP8, BF16, EPI_RELU, 6, NORMAL, NORMAL),
    ]
}


def draw(shape, dist: Dist, dtype: int, gen: torch.Generator) -> torch.Tensor:
    """fp32 draw on the generator's device (the CPU for the workloads), then
    rounded to the 16-bit storage type."""
    dev = gen.device
    if dist.kind == "normal":
        x = torch.randn(shape, generator=gen, dtype=torch.float32, device=dev) * dist.b + dist.a
    elif dist.kind == "randint":
        x = torch.randint(int(dist.a), int(dist.b) + 1, shape, generator=gen, device=dev).to(torch.float32)
    elif dist.kind == "uniform":
        x = torch.rand(shape, generator=gen, dtype=torch.float32, device=dev) * (dist.b - dist.a) + dist.a
    else:
        raise ValueError(dist.kind)
    return x.to(TORCH_DTYPE[dtype])


def make_inputs(w: Workload, seed: int | None = None):
    """(A, B) on the CPU: A is [batch, M, K] (or [M, K]), B is [batch, K, N]."""
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    sa = (w.batch, w.M, w.K) if w.batch > 1 else (w.M, w.K)
    sb = (w.batch, w.K, w.N) if w.batch > 1 else (w.K, w.N)
    A = draw(sa, w.dist_a, w.in_dtype, gen)
    B = draw(sb, w.dist_b, w.in_dtype, gen)
    return A, B


def custom(M, N, K, in_dtype=F16, out_dtype=F32, epilogue=EPI_RELU, dist=NORMAL, seed=0,
           batch=1, dist_b=None, name=None) -> Workload:
    """A small workload for parity cases (same drawing rules as the five)."""
    exact = (dist.kind == "randint" and (dist_b or dist).kind == "randint"
             and epilogue in (EPI_NONE, EPI_RELU))
    return Workload(name or f"custom_{M}x{N}x{K}", M, N, K, in_dtype, out_dtype, epilogue, seed,
                    dist, dist_b or dist, batch=batch, exact=exact)


def draw_bias(N: int, dist: Dist, seed: int) -> torch.Tensor:
    """A bias row of N fp32 values (not rounded to a 16-bit type)."""
    gen = torch.Generator().manual_seed(seed)
    if dist.kind == "normal":
        return torch.randn(N, generator=gen, dtype=torch.float32) * dist.b + dist.a
    if dist.kind == "randint":
        return torch.randint(int(dist.a), int(dist.b) + 1, (N,), generator=gen).to(torch.float32)
    return torch.rand(N, generator=gen, dtype=torch.float32) * (dist.b - dist.a) + dist.a


def sample_indices(M: int, N: int, count: int, seed: int, batch: int = 1):
    """Output positions to check one by one at full size: the four corners,
    the last row and column, and seeded uniform positions."""
    rng = np.random.default_rng(seed)
    fixed = [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]
    fixed += [(M - 1, int(j)) for j in rng.integers(0, N, 8)]
    fixed += [(int(i), N - 1) for i in rng.integers(0, M, 8)]
    n_rand = max(count - len(fixed), 0)
    ii = np.concatenate([np.array([f[0] for f in fixed], np.int64), rng.integers(0, M, n_rand)])
    jj = np.concatenate([np.array([f[1] for f in fixed], np.int64), rng.integers(0, N, n_rand)])
    bi = rng.integers(0, batch, ii.size).astype(np.int64)
    return bi, ii.astype(np.int64), jj.astype(np.int64)
