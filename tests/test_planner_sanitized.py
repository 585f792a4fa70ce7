"""The host side of libtcgemm under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

tests/planner_fuzz.cpp stubs the HIP runtime and the kernel launchers and
feeds seeded random, edge and invalid problem descriptions, device
capabilities, run arguments and tune-cache text to every host entry point
of tensor_core_gemm_amd/csrc/tcgemm_host.cpp (the planner, the run
entry points' argument checks and launch-argument construction, the stage
rule, the tune cache); its stub launchers check the grid and trip
arithmetic the host hands each kernel.  Any sanitizer report or invariant
violation fails the test.  The same harness built under ThreadSanitizer runs
its loop on eight threads at once (the planner's device-capability cache
and the tune cache are shared by every thread of a process).
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_core_gemm_amd", "csrc")


def build_fuzz(d, sanitize):
    out = str(d / "planner_fuzz")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
             "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             *sanitize]
    for src, obj in ((os.path.join(CSRC, "tcgemm_host.cpp"), d / "host.o"),
                     (os.path.join(ROOT, "tests", "planner_fuzz.cpp"), d / "fuzz.o")):
        subprocess.run(["g++", *flags, "-x", "c++", "-c", src, "-o", str(obj)], check=True)
    # gemm_run_noalloc lives in a HIP source with a device array: link a
    # host-only stand-in that makes the same size check and calls
    # gemm_run_ex, so its argument path is exercised too.
    stand_in = d / "noalloc_host.cpp"
    stand_in.write_text(
        '#include "tcgemm.h"\n'
        'extern "C" int gemm_run_noalloc(gemm_plan_t p, const void* A, const void* B, void* C,\n'
        '                                const void* bias, void* s) {\n'
        '  gemm_plan_info in;\n'
        '  int rc = gemm_plan_get_info(p, &in);\n'
        '  if (rc) return rc;\n'
        '  if (in.workspace_bytes > GEMM_NOALLOC_SCRATCH_BYTES) return GEMM_E_SCRATCH;\n'
        '  static char arr[64];\n'
        '  gemm_run_args a = {};\n'
        '  a.bias = bias;\n'
        '  if (in.workspace_bytes > 0) { a.workspace = arr; a.workspace_bytes = GEMM_NOALLOC_SCRATCH_BYTES; }\n'
        '  return gemm_run_ex(p, A, B, C, &a, s);\n'
        '}\n')
    subprocess.run(["g++", *flags, "-c", str(stand_in), "-o", str(d / "noalloc.o")], check=True)
    subprocess.run(["g++", *flags, str(d / "host.o"), str(d / "fuzz.o"), str(d / "noalloc.o"), "-pthread",
                    "-o", out], check=True)
    return out


@pytest.fixture(scope="module")
def fuzz_bin(tmp_path_factory):
    return build_fuzz(tmp_path_factory.mktemp("fuzz"), ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"])


@pytest.fixture(scope="module")
def fuzz_bin_tsan(tmp_path_factory):
    return build_fuzz(tmp_path_factory.mktemp("fuzz_tsan"), ["-fsanitize=thread"])


def test_host_entry_points_under_asan_and_ubsan(fuzz_bin, tmp_path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([fuzz_bin, "30000", str(tmp_path / "cache.txt")], capture_output=True, text=True,
                       env=env, timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    # the run reached the launchers, so the argument paths were exercised
    launches = int(r.stdout.split("stub launches ")[1].split(",")[0])
    assert launches > 100


def test_host_entry_points_from_threads_under_tsan(fuzz_bin_tsan, tmp_path):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    r = subprocess.run([fuzz_bin_tsan, "16000", str(tmp_path / "cache.txt"), "8"], capture_output=True,
                       text=True, env=env, timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "ThreadSanitizer" not in r.stderr
    assert "threads 8" in r.stdout
    launches = int(r.stdout.split("stub launches ")[1].split(",")[0])
    assert launches > 100
