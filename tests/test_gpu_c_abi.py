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


def run_client(w, tmp_path, *extra):
    """Run the C client on w's seeded inputs; returns (A, B, C, stdout)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(CLIENT), "build the library first (it builds the C client too)"
    A, B = gw.make_inputs(w)
    pa, pb, pc = tmp_path / "a.bin", tmp_path / "b.bin", tmp_path / "c.bin"
    pa.write_bytes(raw(A))
    pb.write_bytes(raw(B))
    note(f"C client {w.name} {' '.join(extra)}")
    r = subprocess.run([CLIENT, str(w.M), str(w.N), str(w.K), str(w.in_dtype), str(w.out_dtype),
                        str(w.epilogue), str(pa), str(pb), str(pc), *extra],
                       capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert "plan: tile" in r.stdout and r.stdout.strip().endswith("ok")
    odt = np.float32 if w.out_dtype == F32 else np.uint16
    C = np.frombuffer(pc.read_bytes(), odt).reshape(w.M, w.N)
    return A, B, C, r.stdout


@pytest.mark.parametrize("w", [
    gw.custom(256, 256, 256, F16, F32, EPI_RELU, gw.INT4, seed=1, name="int_f16"),
    gw.custom(300, 200, 130, BF16, BF16, EPI_NONE, gw.NORMAL, seed=2, name="ragged_bf16"),
    gw.custom(130, 96, 256, FP8, F32, EPI_RELU, gw.NORMAL, seed=3, name="fp8"),
    # enough rows for the persistent short-K tile (two 128-row blocks per CU or more)
    gw.custom(70000, 288, 96, F16, F16, EPI_NONE, gw.NORMAL, seed=4, name="short_k_f16",
              dist_b=gw.Dist("normal", 0.0, 96 ** -0.5)),
], ids=lambda w: w.name)
def test_c_client_matches_the_oracle(w, tmp_path):
    A, B, C, out = run_client(w, tmp_path)
    assert "info: split_k 1 tail_rows 0 tail_split 0 workspace 0" in out
    if w.name == "short_k_f16":
        assert "plan: tile 11" in out
    ref, Y = oracle.gemm(A, B, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, want_y=True)
    got = oracle.to_float(w.out_dtype, C)
    if w.exact:
        assert np.array_equal(got, oracle.to_float(w.out_dtype, ref[0]))
    else:
        assert rel_errors(got, Y[0], w.sigma_out()).max() <= TOL


def test_c_client_runs_a_split_tail_plan(tmp_path):
    """GEMM_FLAG_SPLIT_K from C: 4608^3 runs its last 1024 rows as a second
    launch with K split in 3 (on 256 CUs), with the workspace the plan
    asks for; integer inputs, so sampled outputs match the oracle exactly."""
    if torch.cuda.is_available() and torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the tail split of 4608^3 is planned for 256 CUs")
    w = gw.custom(4608, 4608, 4608, F16, F32, EPI_RELU, gw.INT4, seed=5, name="split_tail")
    A, B, C, out = run_client(w, tmp_path, "split")
    assert "tail_rows 1024 tail_split 3" in out
    bi, ii, jj = gw.sample_indices(w.M, w.N, 8192, 5)
    want, _ = oracle.gemm_sampled(A, B, w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, bi, ii, jj)
    assert np.array_equal(C[ii, jj], oracle.to_float(w.out_dtype, want))
