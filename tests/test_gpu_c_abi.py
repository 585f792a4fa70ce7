"""The C ABI used from C: tests/c_abi_check.cpp (built with the library,
linked against libtcgemm.so and the HIP runtime only, no Python or torch)
plans and runs the GEMM in a process of its own; its output is compared
with the CPU oracle here."""
import os
import subprocess

import numpy as np
import pytest
import torch

import gemm_workloads as gw
import oracle
from gemm_workloads import BF16, EPI_NONE, EPI_RELU, F16, F32, FP8
from gpu_helpers import TOL, note, rel_errors

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "tensor_core_gemm_amd", "c_abi_check")


def raw(t):
    t = t.contiguous()
    return t.view(torch.uint8).numpy().tobytes() if t.element_size() == 1 else \
        t.view(torch.int16).numpy().tobytes()


@pytest.mark.parametrize("w", [
    gw.custom(256, 256, 256, F16, F32, EPI_RELU, gw.INT4, seed=1, name="int_f16"),
    gw.custom(300, 200, 130, BF16, BF16, EPI_NONE, gw.NORMAL, seed=2, name="ragged_bf16"),
    gw.custom(130, 96, 256, FP8, F32, EPI_RELU, gw.NORMAL, seed=3, name="fp8"),
    # enough rows for the persistent short-K tile (two 128-row blocks per CU or more)
    gw.custom(70000, 288, 96, F16, F16, EPI_NONE, gw.NORMAL, seed=4, name="short_k_f16",
              dist_b=gw.Dist("normal", 0.0, 96 ** -0.5)),
], ids=lambda w: w.name)
def test_c_client_matches_the_oracle(w, tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(CLIENT), "build the library first (it builds the C client too)"
    A, B = gw.make_inputs(w)
    pa, pb, pc = tmp_path / "a.bin", tmp_path / "b.bin", tmp_path / "c.bin"
    pa.write_bytes(raw(A))
    pb.write_bytes(raw(B))
    note(f"C client {w.name}")
    r = subprocess.run([CLIENT, str(w.M), str(w.N), str(w.K), str(w.in_dtype), str(w.out_dtype),
                        str(w.epilogue), str(pa), str(pb), str(pc)],
                       capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert "plan: tile" in r.stdout and r.stdout.strip().endswith("ok")
    if w.name == "short_k_f16":
        assert "plan: tile 11" in r.stdout
    odt = np.float32 if w.out_dtype == F32 else np.uint16
    C = np.frombuffer(pc.read_bytes(), odt).reshape(w.M, w.N)
    ref, Y = oracle.gemm(A, B, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, want_y=True)
    got = oracle.to_float(w.out_dtype, C)
    if w.exact:
        assert np.array_equal(got, oracle.to_float(w.out_dtype, ref[0]))
    else:
        assert rel_errors(got, Y[0], w.sigma_out()).max() <= TOL
