"""Build libtcgemm.so in place with hipcc for gfx950.

Every source under csrc/ is compiled to an object (in parallel) and linked
into tensor_core_gemm_amd/libtcgemm.so.  All HIP code is built with packed
fp32 instructions disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtcgemm.so")
# A C-ABI client test program (tests/c_abi_check.cpp), linked against the library.
C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_abi_check.cpp")
C_CLIENT = os.path.join(HERE, "c_abi_check")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]


# Per-source flags.  The persistent short-K kernel keeps its accumulators in
# ordinary VGPRs (MFMAs in their VGPR form): its epilogue then reads them
# directly instead of copying every value out of the accumulation registers
# first, which made the epilogue the longest step of each block.
EXTRA = {"tcgemm_shortk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), *(extra or []), "-x", "hip", "-c", src,
               "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out, flush=True)
    if failed:
        for src, out in failed:
            sys.stderr.write(f"--- {src}\n{out}\n")
        raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(s) for s, _ in failed))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if os.path.exists(C_CLIENT_SRC):
        tmp = C_CLIENT + f".tmp{os.getpid()}"
        cmd = [HIPCC, "-O2", "-std=c++17", "-I", INCLUDE, C_CLIENT_SRC, "-L", HERE, "-ltcgemm",
               "-Wl,-rpath,$ORIGIN", "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, C_CLIENT)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
