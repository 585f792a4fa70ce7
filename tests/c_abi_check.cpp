// A C-ABI client of libtcgemm.so that uses nothing but include/tcgemm.h and
// the HIP runtime (no Python, no torch): it reads A and B from files, plans
// and runs C = epilogue(A . B) on device 0, and writes C to a file.  The
// GPU test that runs it compares C with the CPU oracle.
//
// usage: c_abi_check M N K in_dtype out_dtype epilogue a.bin b.bin c.bin
//   (codes as in tcgemm.h; a.bin / b.bin hold the raw operand elements)
// It also checks that the plan and run calls reject bad input with the
// documented codes, and prints the plan description.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "tcgemm.h"

static bool read_file(const char* path, std::vector<unsigned char>& out, size_t bytes) {
  FILE* f = std::fopen(path, "rb");
  if (!f) return false;
  out.resize(bytes);
  const size_t got = std::fread(out.data(), 1, bytes, f);
  std::fclose(f);
  return got == bytes;
}

#define CHECK_HIP(x)                                                    \
  do {                                                                  \
    hipError_t e_ = (x);                                                \
    if (e_ != hipSuccess) {                                             \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_)); \
      return 3;                                                         \
    }                                                                   \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 10 && argc != 11) {
    std::fprintf(stderr, "usage: %s M N K in_dtype out_dtype epilogue a.bin b.bin c.bin [split]\n", argv[0]);
    return 2;
  }
  // "split": let the planner split K (GEMM_FLAG_SPLIT_K) and run with a workspace
  const bool split = argc == 11 && std::strcmp(argv[10], "split") == 0;
  const int64_t M = std::atoll(argv[1]), N = std::atoll(argv[2]), K = std::atoll(argv[3]);
  const int in_dtype = std::atoi(argv[4]), out_dtype = std::atoi(argv[5]), epi = std::atoi(argv[6]);
  const size_t isz = in_dtype == GEMM_FP8 ? 1 : 2, osz = out_dtype == GEMM_F32 ? 4 : 2;
  std::vector<unsigned char> a, b;
  if (!read_file(argv[7], a, (size_t)(M * K) * isz) || !read_file(argv[8], b, (size_t)(K * N) * isz)) {
    std::fprintf(stderr, "cannot read the operands\n");
    return 2;
  }

  // Errors first: a null description, and a run with a null plan.
  gemm_plan_t bad = nullptr;
  if (gemm_plan(nullptr, &bad) != GEMM_E_ARG) return 4;
  if (gemm_run(nullptr, nullptr, nullptr, nullptr, nullptr) != GEMM_E_PLAN) return 4;
  std::printf("errors: %s / %s\n", gemm_strerror(GEMM_E_ARG), gemm_strerror(GEMM_E_PLAN));

  CHECK_HIP(hipSetDevice(0));
  void *dA = nullptr, *dB = nullptr, *dC = nullptr;
  CHECK_HIP(hipMalloc(&dA, a.size()));
  CHECK_HIP(hipMalloc(&dB, b.size()));
  CHECK_HIP(hipMalloc(&dC, (size_t)(M * N) * osz));
  CHECK_HIP(hipMemcpy(dA, a.data(), a.size(), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dB, b.data(), b.size(), hipMemcpyHostToDevice));

  gemm_desc d = {};
  d.M = M;
  d.N = N;
  d.K = K;
  d.in_dtype = in_dtype;
  d.out_dtype = out_dtype;
  d.epilogue = epi;
  d.batch = 1;
  if (split) d.flags = GEMM_FLAG_SPLIT_K;
  gemm_plan_t plan = nullptr;
  int rc = gemm_plan(&d, &plan);
  if (rc != GEMM_OK) {
    std::fprintf(stderr, "gemm_plan: %s\n", gemm_strerror(rc));
    return 5;
  }
  std::printf("plan: %s\n", gemm_plan_describe(plan));
  gemm_plan_info info;
  if (gemm_plan_get_info(plan, &info) != GEMM_OK) return 5;
  std::printf("info: split_k %d tail_rows %lld tail_split %d workspace %lld\n", info.split_k,
              (long long)info.tail_rows, info.tail_split, (long long)info.workspace_bytes);
  void* dW = nullptr;
  if (info.workspace_bytes > 0) CHECK_HIP(hipMalloc(&dW, (size_t)info.workspace_bytes));
  gemm_run_args args = {};
  args.workspace = dW;
  args.workspace_bytes = info.workspace_bytes;
  // C overlapping A is refused before anything runs.
  if (gemm_run_ex(plan, dA, dB, dA, &args, nullptr) != GEMM_E_ALIAS) return 4;

  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));
  rc = gemm_run_ex(plan, dA, dB, dC, &args, s);
  if (rc != GEMM_OK) {
    std::fprintf(stderr, "gemm_run: %s\n", gemm_strerror(rc));
    return 5;
  }
  CHECK_HIP(hipStreamSynchronize(s));
  std::vector<unsigned char> c((size_t)(M * N) * osz);
  CHECK_HIP(hipMemcpy(c.data(), dC, c.size(), hipMemcpyDeviceToHost));
  FILE* f = std::fopen(argv[9], "wb");
  if (!f || std::fwrite(c.data(), 1, c.size(), f) != c.size()) return 2;
  std::fclose(f);
  gemm_plan_destroy(plan);
  CHECK_HIP(hipStreamDestroy(s));
  CHECK_HIP(hipFree(dA));
  CHECK_HIP(hipFree(dB));
  CHECK_HIP(hipFree(dC));
  if (dW) CHECK_HIP(hipFree(dW));
  std::printf("ok\n");
  return 0;
}
