"""Mutation check of the oracle's pins (run by hand: python3 tests/oracle_mutants.py).

Applies one plausible slip at a time to a copy of oracle/oracle.c in a
temporary directory (a changed constant, sign, index, comparison, rounding
rule, stride or loop bound), builds that copy, and runs the oracle's CPU
tests against it.  A mutant that no test fails is reported as a survivor.
The repository's own oracle is never modified.

Two mutants are known to be equivalent and survive by construction:
"relu >=" differs from the oracle only on -0, which the fold never produces
(it starts at +0, and in round-to-nearest x + (-x) is +0);
"f64 S signed" computes |a b| instead of |a| |b|, equal in double because
the product of two 16-bit values is exact there.

Usage: python3 tests/oracle_mutants.py [mutant names...]
"""
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

M = [
    ("f16 dec subnormal scale", "ldexpf((float)f, -24)", "ldexpf((float)f, -25)"),
    ("f16 dec normal exp", "ldexpf((float)(1024 + f), e - 25)", "ldexpf((float)(1024 + f), e - 24)"),
    ("f16 dec inf->nan", "if (f == 0) {\n      v = INFINITY;", "if (f == 1) {\n      v = INFINITY;"),
    ("f16 dec sign", "  return sign ? -v : v;\n}\n\n/* bfloat16", "  return v;\n}\n\n/* bfloat16"),
    ("bf16 dec shift", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    ("fp8 nan any frac", "if (e == 15 && f == 7) {", "if (e == 15) {"),
    ("fp8 subnormal", "v = ldexpf((float)f, -9);", "v = ldexpf((float)f, -10);"),
    ("fp8 normal exp", "ldexpf((float)(8 + f), e - 10)", "ldexpf((float)(8 + f), e - 11)"),
    ("fp8 sign", "  return sign ? -v : v;\n}\n\n/* Element idx", "  return v;\n}\n\n/* Element idx"),
    ("rne ties up", "if (rem > half || (rem == half && (q & 1u))) q += 1u;", "if (rem >= half) q += 1u;"),
    ("rne ties odd", "(rem == half && (q & 1u))", "(rem == half && !(q & 1u))"),
    ("rne truncate", "if (rem > half || (rem == half && (q & 1u))) q += 1u;", ""),
    ("f16 enc shift>=32", "if (shift >= 32) return 0;", "if (shift >= 32) return 1;"),
    ("f16 enc nan test", "if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u", "if (a >= 0x7f800000u) return (uint16_t)(sign | 0x7e00u"),
    ("f16 enc nan quiet", "sign | 0x7e00u | ((a >> 13) & 0x1ffu)", "sign | 0x7c00u | ((a >> 13) & 0x1ffu)"),
    ("f16 enc quantum", "int q_exp = (unb < -14) ? -24 : unb - 10;", "int q_exp = (unb < -14) ? -24 : unb - 11;"),
    ("f16 enc subnormal bound", "int q_exp = (unb < -14) ? -24", "int q_exp = (unb < -15) ? -24"),
    ("f16 enc carry", "if (q >= 2048u) { q >>= 1; E += 1; }", "if (q > 2048u) { q >>= 1; E += 1; }"),
    ("f16 enc overflow", "if (E > 15) return (uint16_t)(sign | 0x7c00u);", "if (E > 16) return (uint16_t)(sign | 0x7c00u);"),
    ("f16 enc bias", "(uint16_t)((E + 15) << 10)", "(uint16_t)((E + 14) << 10)"),
    ("f16 enc subnormal mask", "return (uint16_t)(sign | q); /* q <= 1024", "return (uint16_t)(sign | (q & 1023u)); /* q <= 1024"),
    ("bf16 enc ties up", "if (rem > 0x8000u || (rem == 0x8000u && (hi & 1u))) hi += 1u;", "if (rem >= 0x8000u) hi += 1u;"),
    ("bf16 enc truncate", "if (rem > 0x8000u || (rem == 0x8000u && (hi & 1u))) hi += 1u;", ""),
    ("bf16 enc nan quiet", "return (uint16_t)((u >> 16) | 0x0040u);", "return (uint16_t)((u >> 16));"),
    ("relu >=", "return (v > 0.0f) ? v : 0.0f;", "return (v >= 0.0f) ? v : 0.0f;"),
    ("relu -0", "return (v > 0.0f) ? v : 0.0f;", "return (v > 0.0f) ? v : -0.0f;"),
    ("relu nan passes", "return (v > 0.0f) ? v : 0.0f;", "return (v <= 0.0f) ? 0.0f : v;"),
    ("gelu half", "case 2: return (float)(0.5 * x", "case 2: return (float)(0.49 * x"),
    ("gelu cubic coef", "(x + 0.044715 * x", "(x + 0.0447 * x"),
    ("gelu sqrt", "tanh(sqrt(2.0 / pi)", "tanh(1.001 * sqrt(2.0 / pi)"),
    ("gelu cube->square", "0.044715 * x * x * x", "0.044715 * x * x"),
    ("gelu_erf arg", "erf(x / sqrt(2.0))", "erf(x / sqrt(2.1))"),
    ("gelu_erf half", "case 3: return (float)(0.5 * x", "case 3: return (float)(0.51 * x"),
    ("sigmoid sign", "exp(-x)", "exp(x)"),
    ("sigmoid one", "(1.0 / (1.0 + exp(-x)))", "(1.0 / (1.01 + exp(-x)))"),
    ("tanh scale", "default: return (float)tanh(x);", "default: return (float)tanh(1.0001 * x);"),
    ("tanh fp32", "default: return (float)tanh(x);", "default: return tanhf(v);"),
    ("gelu fp32", "case 2: return (float)(0.5 * x * (1.0 + tanh(sqrt(2.0 / pi) * (x + 0.044715 * x * x * x))));",
     "case 2: return 0.5f * v * (1.0f + tanhf(0.7978845608f * (v + 0.044715f * v * v * v)));"),
    ("bias minus", "bias ? acc + bias[j] : acc", "bias ? acc - bias[j] : acc"),
    ("bias wrong col", "bias ? acc + bias[j] : acc", "bias ? acc + bias[0] : acc"),
    ("bias after act", "const float v = bias ? acc + bias[j] : acc;\n  return orc_activate(v, act);",
     "const float y = orc_activate(acc, act);\n  return bias ? y + bias[j] : y;"),
    ("store f16<->bf16", "((uint16_t*)C)[idx] = orc_f16_encode(y);\n  else\n    ((uint16_t*)C)[idx] = orc_bf16_encode(y);",
     "((uint16_t*)C)[idx] = orc_bf16_encode(y);\n  else\n    ((uint16_t*)C)[idx] = orc_f16_encode(y);"),
    ("gemm init -0", "for (int64_t j = 0; j < N; ++j) acc[j] = 0.0f;", "for (int64_t j = 0; j < N; ++j) acc[j] = -0.0f;"),
    ("gemm drop last k", "      for (int64_t k = 0; k < K; ++k) {\n        const float a = af[i * K + k];",
     "      for (int64_t k = 0; k < K - 1; ++k) {\n        const float a = af[i * K + k];"),
    ("gemm reversed k", "const float a = af[i * K + k];\n        const float* brow = bf + k * N;",
     "const float a = af[i * K + (K - 1 - k)];\n        const float* brow = bf + (K - 1 - k) * N;"),
    ("gemm fma", "acc[j] = acc[j] + a * brow[j];", "acc[j] = fmaf(a, brow[j], acc[j]);"),
    ("gemm double acc", "acc[j] = acc[j] + a * brow[j];", "acc[j] = (float)((double)acc[j] + (double)a * (double)brow[j]);"),
    ("gemm B stride", "orc_decode_batch(in_dtype, B, b * stride_b, bf, K * N);\n    int64_t i;\n#pragma omp parallel for schedule(dynamic, 1)\n    for (i = 0; i < M; ++i) {\n      float* acc",
     "orc_decode_batch(in_dtype, B, b * stride_a, bf, K * N);\n    int64_t i;\n#pragma omp parallel for schedule(dynamic, 1)\n    for (i = 0; i < M; ++i) {\n      float* acc"),
    ("gemm C stride", "orc_store(out_dtype, C, b * stride_c + i * N + j, y);", "orc_store(out_dtype, C, b * M * N + i * N + j, y);"),
    ("gemm transposed B", "const float* brow = bf + k * N;\n        for (int64_t j = 0; j < N; ++j) acc[j] = acc[j] + a * brow[j];",
     "for (int64_t j = 0; j < N; ++j) acc[j] = acc[j] + a * bf[(j % K) * N + (k % N)];"),
    ("sampled col index", "float bv = orc_decode_at(in_dtype, B, bcol + k * N);", "float bv = orc_decode_at(in_dtype, B, bcol + k * N - (k > 0));"),
    ("sampled batch", "const int64_t arow = bi[e] * stride_a + ii[e] * K;", "const int64_t arow = ii[e] * K;"),
    ("sampled bias col", "float y = orc_epilogue(acc, bias, jj[e], epilogue);", "float y = orc_epilogue(acc, bias, ii[e] % N, epilogue);"),
    ("sampled drop last k", "for (int64_t k = 0; k < K; ++k) {\n      float a = orc_decode_at", "for (int64_t k = 0; k + 1 < K; ++k) {\n      float a = orc_decode_at"),
    ("f64 S doubled", "sab[j] = sab[j] + fabs(a) * fabs((double)brow[j]);", "sab[j] = sab[j] + 2.0 * fabs(a) * fabs((double)brow[j]);"),
    ("f64 S signed", "sab[j] = sab[j] + fabs(a) * fabs((double)brow[j]);", "sab[j] = sab[j] + fabs(a * (double)brow[j] + 0.0 * a);"),
    ("f64 Y float", "acc[j] = acc[j] + a * (double)brow[j];", "acc[j] = (float)(acc[j] + a * (double)brow[j]);"),
    ("f64 S no abs b", "fabs(a) * fabs((double)brow[j])", "fabs(a) * (double)brow[j]"),
    ("check epi range", "if (epilogue < 0 || epilogue > 5) return ORC_EARG;", "if (epilogue < 0 || epilogue > 4) return ORC_EARG;"),
    ("check fp8 out", "if (out_dtype != ORC_F32 && out_dtype != ORC_F16 && out_dtype != ORC_BF16) return ORC_EDTYPE;",
     "if (out_dtype != ORC_F32 && out_dtype != ORC_F16 && out_dtype != ORC_BF16 && out_dtype != ORC_FP8) return ORC_EDTYPE;"),
    ("K=0 output", "  if (M == 0 || N == 0) return ORC_OK;\n  orc_set_threads(threads);\n  float* bf = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K * N : 1));\n  float* af = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? M * K : 1));\n  if (!bf || !af) { free(bf); free(af); return ORC_ENOMEM; }\n  for (int64_t b = 0; b < batch; ++b) {\n    orc_decode_batch(in_dtype, A, b * stride_a, af, M * K);\n    orc_decode_batch(in_dtype, B, b * stride_b, bf, K * N);\n    int64_t i;\n#pragma omp parallel for schedule(dynamic, 1)\n    for (i = 0; i < M; ++i) {\n      float* acc",
     "  if (M == 0 || N == 0 || K == 0) return ORC_OK;\n  orc_set_threads(threads);\n  float* bf = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K * N : 1));\n  float* af = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? M * K : 1));\n  if (!bf || !af) { free(bf); free(af); return ORC_ENOMEM; }\n  for (int64_t b = 0; b < batch; ++b) {\n    orc_decode_batch(in_dtype, A, b * stride_a, af, M * K);\n    orc_decode_batch(in_dtype, B, b * stride_b, bf, K * N);\n    int64_t i;\n#pragma omp parallel for schedule(dynamic, 1)\n    for (i = 0; i < M; ++i) {\n      float* acc"),
]

TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_epilogue.py", "tests/test_oracle_fp8.py"]


def setup(WORK):
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(WORK, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.so"))
    shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(WORK, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "gemm_workloads.py"), WORK)


def main():
    WORK = tempfile.mkdtemp(prefix="oracle_mutants_")
    try:
        return sweep(WORK)
    finally:
        shutil.rmtree(WORK, ignore_errors=True)


def sweep(WORK):
    setup(WORK)
    src0 = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    only = sys.argv[1:]
    survivors = []
    for name, old, new in M:
        if only and name not in only:
            continue
        n = src0.count(old)
        if n != 1:
            print(f"!! {name}: pattern found {n} times", flush=True)
            continue
        open(os.path.join(WORK, "oracle", "oracle.c"), "w").write(src0.replace(old, new))
        lib = os.path.join(WORK, "oracle", "liboracle.so")
        if os.path.exists(lib):
            os.remove(lib)
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *TESTS],
                           cwd=WORK, capture_output=True, text=True, timeout=600)
        killed = r.returncode != 0
        last = (r.stdout.strip().splitlines() or ["?"])[-1]
        print(f"{'caught  ' if killed else 'SURVIVED'} {name}: {last}", flush=True)
        if not killed:
            survivors.append(name)
    print("survivors:", survivors)
    known = {"relu >=", "f64 S signed"}
    return 0 if set(survivors) <= known else 1


if __name__ == "__main__":
    sys.exit(main())
