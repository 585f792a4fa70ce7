// A CPU harness for the host side of libtcgemm (tcgemm_host.cpp), built with
// g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_planner_sanitized.py.  The HIP runtime and the kernel
// launchers are replaced by stubs defined here, so nothing runs on a GPU:
// the stubs either report no device, or a gfx950 with 256 CUs whose
// "launches" only check the arguments the host built for them.
//
// A seeded generator draws problem descriptions (valid, edge and invalid
// sizes, strides, types, flags, tiles and splits), device capabilities,
// run arguments and tune-cache text, and feeds them to every host entry
// point.  Any sanitizer report aborts the process; the harness itself
// checks a few invariants of the plans and the launch arguments and exits
// non-zero on a violation.  With a thread count (third argument) the same
// loop runs on that many threads at once, each with its own generator, so
// that a ThreadSanitizer build sees the planner, the run entry points and
// the tune cache used concurrently.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <string>
#include <thread>
#include <vector>

#include "tcgemm.h"
#include "tcgemm_kernel_args.h"
#include "tcgemm_tiles.h"

// ---------------------------------------------------------------------------
// Stubs of the HIP runtime calls the host code makes.
static thread_local bool g_device = false;  // pretend a gfx950 is present
static std::atomic<long> g_launches{0};
static std::atomic<int> g_failures{0};
static uint64_t next();

#define FAIL(...)                         \
  do {                                    \
    fprintf(stderr, "invariant: ");       \
    fprintf(stderr, __VA_ARGS__);         \
    fprintf(stderr, "\n");                \
    ++g_failures;                         \
  } while (0)

extern "C" {
hipError_t hipGetDevice(int* d) {
  if (!g_device) return hipErrorNoDevice;
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetDeviceCount(int* n) {
  *n = g_device ? 1 : 0;
  return g_device ? hipSuccess : hipErrorNoDevice;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* p, int d) {
  if (!g_device || d != 0) return hipErrorInvalidDevice;
  memset(p, 0, sizeof(*p));
  snprintf(p->gcnArchName, sizeof(p->gcnArchName), "gfx950:sramecc+:xnack-");
  p->multiProcessorCount = 256;
  p->warpSize = 64;
  p->clockRate = 2400000;
  p->sharedMemPerBlock = 163840;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 163840;
  return g_device ? hipSuccess : hipErrorNoDevice;
}
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = reinterpret_cast<hipEvent_t>(new int(0));
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
  delete reinterpret_cast<int*>(e);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.1f + (float)(next() % 100) * 0.001f;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipRuntimeGetVersion(int* v) {
  *v = 70000000;
  return hipSuccess;
}
}

// ---------------------------------------------------------------------------
// Stub launchers: check what a kernel would be given.
static void check_kargs(int tile, const tcg::KArgs& a) {
  ++g_launches;
  const tcg::TileDesc& t = tcg::kTiles[tile - 1];
  const int64_t nt = (int64_t)t.wm * t.wn * 64;
  if (a.workgroups <= 0 || a.workgroups * nt >= ((int64_t)1 << 32)) FAIL("tile %d: workgroups %lld", tile, (long long)a.workgroups);
  if (a.M <= 0 || a.N <= 0 || a.K < 0) FAIL("tile %d: empty launch", tile);
  if (a.splits < 1 || a.trips_per_split < 0 || (int64_t)a.splits * a.trips_per_split < a.trips)
    FAIL("tile %d: splits %d x %d trips < %d", tile, a.splits, a.trips_per_split, a.trips);
  if (a.splits > 1 && !a.ws) FAIL("tile %d: split without workspace", tile);
  if (!t.persistent && a.workgroups != a.tiles_m * a.tiles_n * a.batch * a.splits)
    FAIL("tile %d: grid %lld != %lld x %lld x %lld x %d", tile, (long long)a.workgroups, (long long)a.tiles_m,
         (long long)a.tiles_n, (long long)a.batch, a.splits);
  if (!t.persistent && (a.tiles_m * t.bm < a.M || a.tiles_n * t.bn < a.N)) FAIL("tile %d: grid misses C", tile);
  if ((int64_t)t.bm * (a.K > 0 ? a.K : 1) * t.esize >= 0x7fffffff) FAIL("tile %d: A offsets beyond 31 bits", tile);
}
namespace tcg {
#define STUB(n)                                                                  \
  hipError_t launch_t##n(int, bool, bool, const KArgs& a, hipStream_t) {         \
    check_kargs(n, a);                                                           \
    return hipSuccess;                                                           \
  }                                                                              \
  hipError_t launch_t##n##_gen(int, bool, bool, const KArgs& a, hipStream_t) {  \
    check_kargs(n, a);                                                           \
    return hipSuccess;                                                           \
  }
STUB(1)
STUB(2)
STUB(3)
STUB(4)
STUB(5)
STUB(6)
STUB(7)
STUB(8)
STUB(9)
STUB(10)
STUB(12)
STUB(13)
#undef STUB
hipError_t launch_t11(bool, const KArgs& a, hipStream_t) {
  check_kargs(11, a);
  return hipSuccess;
}
hipError_t launch_splitk_reduce(const RArgs& r, hipStream_t) {
  if (r.splits < 2 || !r.ws || !r.C || r.M <= 0 || r.N <= 0) FAIL("reduce: splits %d", r.splits);
  return hipSuccess;
}
}  // namespace tcg

// ---------------------------------------------------------------------------
static thread_local uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t next() {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return g_rng;
}
static int64_t pick(const int64_t* v, int n) { return v[next() % n]; }

static int64_t draw_size() {
  static const int64_t edge[] = {0, 1, 2, 3, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127,
                                 128, 129, 255, 256, 257, 288, 1000, 1024, 4096, 16384, 129600, -1, -7,
                                 (int64_t)1 << 20, (int64_t)1 << 31, ((int64_t)1 << 31) + 8, (int64_t)1 << 40,
                                 INT64_MAX};
  switch (next() % 4) {
    case 0: return pick(edge, sizeof(edge) / sizeof(edge[0]));
    case 1: return (int64_t)(next() % 5000);
    case 2: return 8 * (int64_t)(next() % 2048);
    default: return (int64_t)(next() % 300000);
  }
}

static gemm_desc draw_desc() {
  static const int64_t dtypes[] = {GEMM_F32, GEMM_F16, GEMM_BF16, GEMM_FP8, 1, 7, -1};
  gemm_desc d;
  memset(&d, 0, sizeof(d));
  d.M = draw_size();
  d.N = draw_size();
  d.K = draw_size();
  d.in_dtype = (int32_t)pick(dtypes, 7);
  d.out_dtype = (int32_t)pick(dtypes, 7);
  d.epilogue = (int32_t)(next() % 8) - 1;
  d.flags = (int32_t)(next() % 128);
  if (next() % 4 == 0) d.flags |= (int32_t)(next() & 0xffff);
  d.batch = next() % 5 == 0 ? draw_size() : 1 + (int64_t)(next() % 4);
  // (products of huge sizes wrap: unsigned arithmetic, then reinterpreted)
  auto prod = [](int64_t x, int64_t y) { return (int64_t)((uint64_t)x * (uint64_t)y + next() % 64); };
  d.stride_a = next() % 3 ? prod(d.M, d.K) : draw_size();
  d.stride_b = next() % 3 ? prod(d.K, d.N) : draw_size();
  d.stride_c = next() % 3 ? prod(d.M, d.N) : draw_size();
  d.tile = next() % 3 ? 0 : (int32_t)(next() % 18) - 2;
  d.split_k = next() % 3 ? 0 : (int32_t)(next() % 300) - 2;
  if (next() % 2) {
    // a valid description: every field in range, sizes from the same mix
    static const int32_t ins[] = {GEMM_F16, GEMM_BF16, GEMM_FP8};
    static const int32_t outs[] = {GEMM_F32, GEMM_F16, GEMM_BF16};
    d.M = d.M < 0 ? 0 : d.M % 70000;
    d.N = d.N < 0 ? 0 : d.N % 70000;
    d.K = d.K < 0 ? 0 : d.K % 70000;
    d.in_dtype = ins[next() % 3];
    d.out_dtype = outs[next() % 3];
    d.epilogue = (int32_t)(next() % 6);
    d.flags = (int32_t)(next() % 64);
    d.batch = 1 + (int64_t)(next() % 3);
    d.stride_a = d.M * d.K + (int64_t)(next() % 3) * 8;
    d.stride_b = d.K * d.N + (int64_t)(next() % 3) * 8;
    d.stride_c = d.M * d.N + (int64_t)(next() % 3) * 8;
    d.tile = 0;
    if (next() % 3 == 0) {
      const int t = 1 + (int)(next() % tcg::kNumTiles);
      if ((tcg::kTiles[t - 1].esize == 1) == (d.in_dtype == GEMM_FP8)) d.tile = t;
    }
    d.split_k = next() % 3 ? 0 : (int32_t)(next() % 20);
  }
  return d;
}

static gemm_device_caps draw_caps() {
  static const int64_t cus[] = {0, 1, 8, 80, 256, 304, -4};
  static const int64_t lds[] = {0, 16, 32768, 65536, 131072, 163840, -1, 1 << 30};
  gemm_device_caps c;
  memset(&c, 0, sizeof(c));
  c.num_cus = (int32_t)pick(cus, 7);
  c.lds_bytes = (int32_t)pick(lds, 8);
  c.async_copy = (int32_t)(next() % 2);
  c.wave_size = next() % 5 ? 64 : 32;
  c.clock_khz = 2400000;
  c.num_xcds = next() % 2 ? 8 : 1;
  snprintf(c.arch, sizeof(c.arch), "%s", next() % 4 ? "gfx950:sramecc+:xnack-" : "gfx942");
  return c;
}

static void check_plan(gemm_plan_t p, const gemm_desc& d, const gemm_device_caps& c) {
  gemm_plan_info in;
  if (gemm_plan_get_info(p, &in) != GEMM_OK) FAIL("get_info on a valid plan");
  const char* text = gemm_plan_describe(p);
  if (!text || strlen(text) == 0 || strlen(text) > 1000) FAIL("describe");
  if (in.tile_id < 1 || in.tile_id > tcg::kNumTiles) FAIL("tile id %d", in.tile_id);
  if (in.lds_bytes > c.lds_bytes) FAIL("plan needs %d B of LDS, device has %d", in.lds_bytes, c.lds_bytes);
  if (in.stages < 0 || in.stages > 4) FAIL("stages %d", in.stages);
  if (in.split_k < 1 || in.workspace_bytes < 0) FAIL("split %d ws %lld", in.split_k, (long long)in.workspace_bytes);
  if (in.split_k > 1 && in.workspace_bytes < (int64_t)in.split_k * d.M * d.N * 4 * (d.batch > 0 ? 1 : 0))
    FAIL("workspace %lld for %d ranges of %lld x %lld", (long long)in.workspace_bytes, in.split_k, (long long)d.M,
         (long long)d.N);
}

static void try_runs(gemm_plan_t p, const gemm_desc& d) {
  gemm_plan_info in;
  gemm_plan_get_info(p, &in);
  // Fake, well-separated device addresses: the host only compares and
  // offsets them before the (stubbed) launch.
  const uintptr_t base = (uintptr_t)1 << 44;
  const void* A = (const void*)(base);
  const void* B = (const void*)(base + ((uintptr_t)1 << 42));
  void* C = (void*)(base + ((uintptr_t)2 << 42));
  void* W = (void*)(base + ((uintptr_t)3 << 42));
  const void* bias = (const void*)(base + ((uintptr_t)3 << 42) + ((uintptr_t)1 << 41));
  gemm_run_args args;
  memset(&args, 0, sizeof(args));
  args.bias = next() % 2 ? bias : nullptr;
  args.workspace = next() % 3 ? W : nullptr;
  args.workspace_bytes = next() % 2 ? in.workspace_bytes : (int64_t)(next() % 1000);
  if (next() % 7 == 0) args.reserved[next() % 4] = 1;
  (void)gemm_run(p, A, B, C, nullptr);
  (void)gemm_run_ex(p, A, B, C, next() % 5 ? &args : nullptr, nullptr);
  (void)gemm_run_ex(p, nullptr, B, C, &args, nullptr);
  (void)gemm_run_ex(p, A, B, (void*)A, &args, nullptr);  // C on A: must be refused, never launched
  (void)gemm_run_noalloc(p, A, B, C, args.bias, nullptr);
  (void)d;
}

// One thread's share of the iterations; tmp: its tune-cache file.
static long fuzz_loop(long iters, const std::string& tmp_s, long offset) {
  const char* tmp = tmp_s.c_str();
  long plans = 0;
  for (long it = 0; it < iters; ++it) {
    g_device = ((it + offset) % 2) == 1;
    gemm_desc d = draw_desc();
    gemm_device_caps c = draw_caps();
    gemm_plan_t p = nullptr;
    const int rc = gemm_plan_for_caps(next() % 50 ? &d : nullptr, next() % 50 ? &c : nullptr, &p);
    if (rc == GEMM_OK) {
      if (!p) FAIL("GEMM_OK with no plan");
      ++plans;
      check_plan(p, d, c);
      try_runs(p, d);
      gemm_plan_destroy(p);
    } else if (p) {
      FAIL("error %d with a plan", rc);
    }
    // the device planner (stub device or none)
    p = nullptr;
    if (gemm_plan(&d, &p) == GEMM_OK) {
      try_runs(p, d);
      gemm_plan_destroy(p);
    }
    // the autotuner on stub launches and events (it fills the tune cache)
    if (it % 53 == 0 && g_device) {
      const uintptr_t base = (uintptr_t)1 << 44;
      gemm_plan_t q = nullptr;
      if (gemm_autotune(&d, (const void*)base, (const void*)(base + ((uintptr_t)1 << 42)),
                        (void*)(base + ((uintptr_t)2 << 42)), nullptr, nullptr, &q) == GEMM_OK)
        gemm_plan_destroy(q);
    }
    // the stage rule on random tiles
    int64_t tiles[3] = {(int64_t)(next() % 200000) - 8, (int64_t)(next() % 200000), (int64_t)(next() % 64)};
    const int st = gemm_stage_depth(&c, (int64_t)(next() % 300000) - 1000, tiles, (int)(next() % 4),
                                    (int)(next() % 2));
    if (st < 0 || st > 2) FAIL("stage depth %d", st);
    (void)gemm_strerror((int)(next() % 40) - 30);
    // tune-cache text: valid and garbled lines
    if (it % 97 == 0) {
      FILE* f = fopen(tmp, "w");
      if (f) {
        for (int l = 0; l < 5; ++l) {
          char line[600];
          if (next() % 2)
            snprintf(line, sizeof(line), "gfx950:sramecc+:xnack- 256 %lld %lld %lld %d %d %d %d %lld %lld %lld %lld %d %d %f\n",
                     (long long)d.M, (long long)d.N, (long long)d.K, d.in_dtype, d.out_dtype, d.epilogue, d.flags,
                     (long long)d.batch, (long long)d.stride_a, (long long)d.stride_b, (long long)d.stride_c,
                     (int)(next() % 16) - 1, (int)(next() % 20) - 1, 1.5);
          else {
            const int n = (int)(next() % (sizeof(line) - 1));
            for (int k = 0; k < n; ++k) line[k] = (char)(32 + next() % 95);
            line[n] = '\n';
            line[n + 1 < (int)sizeof(line) ? n + 1 : n] = 0;
          }
          fputs(line, f);
        }
        fclose(f);
      }
      (void)gemm_tune_cache_load(tmp);
      (void)gemm_tune_cache_save(tmp);
      (void)gemm_tune_cache_size();
      gemm_desc t = d;
      t.flags |= GEMM_FLAG_TUNED;
      gemm_plan_t q = nullptr;
      if (gemm_plan_for_caps(&t, &c, &q) == GEMM_OK) gemm_plan_destroy(q);
      if (next() % 3 == 0) gemm_tune_cache_clear();
    }
  }
  return plans;
}

int main(int argc, char** argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 20000;
  const std::string tmp = argc > 2 ? argv[2] : "/tmp/tcgemm_fuzz_cache.txt";
  const int threads = argc > 3 ? atoi(argv[3]) : 1;
  long plans = 0;
  if (threads <= 1) {
    plans = fuzz_loop(iters, tmp, 0);
  } else {
    std::vector<std::thread> pool;
    std::vector<long> counts(threads, 0);
    for (int i = 0; i < threads; ++i)
      pool.emplace_back([&, i]() {
        g_rng = 0x9E3779B97F4A7C15ull ^ (0x100000001B3ull * (uint64_t)(i + 1));
        counts[i] = fuzz_loop(iters / threads, tmp + "." + std::to_string(i), i);
      });
    for (auto& t : pool) t.join();
    for (long c : counts) plans += c;
  }
  gemm_tune_cache_clear();
  gemm_plan_destroy(nullptr);
  printf("iterations %ld, threads %d, plans %ld, stub launches %ld, invariant failures %d\n", iters, threads, plans,
         g_launches.load(), g_failures.load());
  return g_failures.load() == 0 ? 0 : 1;
}
