// Host side of libtcgemm.so: device capabilities, the planner (tile and
// stage choice) and the C ABI declared in tcgemm.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>

#include "tcgemm.h"
#include "tcgemm_launch.h"
#include "tcgemm_tiles.h"

namespace {

constexpr uint32_t kPlanMagic = 0x7C6E3A11u;
constexpr int kMaxSplits = 256;

struct Plan {
  uint32_t magic;
  gemm_desc d;
  gemm_plan_info info;
  int32_t group_m;
  int32_t xcd_remap;
  char text[560];
  // A plan with a split tail: the unsplit rows above it and the tail rows
  // (owned; both null otherwise).
  Plan* head;
  Plan* tail;
};

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("TCGEMM_LOG");
    return e && *e && *e != '0';
  }();
  return on;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int out_size(int dtype) { return dtype == GEMM_F32 ? 4 : 2; }
int in_size(int dtype) { return dtype == GEMM_FP8 ? 1 : 2; }

const tcg::TileDesc& tile_desc(int id) { return tcg::kTiles[id - 1]; }

// Per-device capability cache.
constexpr int kMaxDevices = 64;
std::mutex g_caps_mu;
bool g_caps_valid[kMaxDevices];
gemm_device_caps g_caps[kMaxDevices];
int g_caps_rc[kMaxDevices];

int cached_caps(int device, gemm_device_caps* out) {
  if (device < 0 || device >= kMaxDevices) return GEMM_E_DEVICE;
  std::lock_guard<std::mutex> lk(g_caps_mu);
  if (!g_caps_valid[device]) {
    g_caps_rc[device] = gemm_device_caps_query(device, &g_caps[device]);
    g_caps_valid[device] = true;
  }
  *out = g_caps[device];
  return g_caps_rc[device];
}

bool is_gfx950(const gemm_device_caps& c) { return std::strncmp(c.arch, "gfx950", 6) == 0; }

// Largest byte extent of one operand over all its batch items.  Every size
// the host derives (extents, offsets, workspaces of up to kMaxSplits ranges,
// grid sizes) stays far inside int64 below it, so no size arithmetic
// overflows; 2^52 bytes is beyond any device's memory.
constexpr int64_t kMaxExtentBytes = (int64_t)1 << 52;

// Bytes spanned by `batch` items of rows x cols elements, `stride` elements
// apart, or -1 if that is not below kMaxExtentBytes.
int64_t extent_bytes(int64_t batch, int64_t stride, int64_t rows, int64_t cols, int64_t esize) {
  int64_t item = 0, span = 0, total = 0, bytes = 0;
  if (__builtin_mul_overflow(rows, cols, &item) || __builtin_mul_overflow(batch - 1, stride, &span) ||
      __builtin_add_overflow(item, span, &total) || __builtin_mul_overflow(total, esize, &bytes) ||
      bytes >= kMaxExtentBytes)
    return -1;
  return bytes;
}

int validate_desc(const gemm_desc* d) {
  if (!d) return GEMM_E_ARG;
  if (d->M < 0 || d->N < 0 || d->K < 0 || d->batch < 1) return GEMM_E_ARG;
  if (d->in_dtype != GEMM_F16 && d->in_dtype != GEMM_BF16 && d->in_dtype != GEMM_FP8) return GEMM_E_DTYPE;
  if (d->out_dtype != GEMM_F32 && d->out_dtype != GEMM_F16 && d->out_dtype != GEMM_BF16)
    return GEMM_E_DTYPE;
  // Each operand's extent, with the strides a run will use (one item: none).
  const int64_t sa = d->batch > 1 ? d->stride_a : 0, sb = d->batch > 1 ? d->stride_b : 0,
                sc = d->batch > 1 ? d->stride_c : 0;
  if (d->batch > 1 && (sa < 0 || sb < 0 || sc < 0)) return GEMM_E_ARG;
  if (extent_bytes(d->batch, sa, d->M, d->K, in_size(d->in_dtype)) < 0 ||
      extent_bytes(d->batch, sb, d->K, d->N, in_size(d->in_dtype)) < 0 ||
      extent_bytes(d->batch, sc, d->M, d->N, 4) < 0)
    return GEMM_E_SIZE;
  if (d->epilogue < GEMM_EPI_NONE || d->epilogue > GEMM_EPI_TANH) return GEMM_E_ARG;
  if (d->flags & ~(GEMM_FLAG_FORCE_STAGES_1 | GEMM_FLAG_UNSTAGED | GEMM_FLAG_FORCE_STAGES_2 |
                   GEMM_FLAG_BIAS | GEMM_FLAG_SPLIT_K | GEMM_FLAG_TUNED))
    return GEMM_E_ARG;
  if (d->tile < 0 || d->tile > tcg::kNumTiles) return GEMM_E_ARG;
  // A tile is built for one operand width: 16-bit tiles for F16/BF16, 8-bit for FP8.
  if (d->tile && tcg::kTiles[d->tile - 1].esize != in_size(d->in_dtype)) return GEMM_E_ARG;
  if (d->split_k < 0 || d->split_k > kMaxSplits) return GEMM_E_ARG;
  if (d->batch > 1) {
    if (d->stride_a < d->M * d->K || d->stride_b < d->K * d->N || d->stride_c < d->M * d->N)
      return GEMM_E_ARG;
  }
  return GEMM_OK;
}

// Time model of the planner, in microseconds, fitted to steady-state timings
// on MI355X (bf16, a sweep of 20 shapes from 512^3 to 8192^3 and skinny,
// deep-K and short-K ones; the FP8 tiles move the same bytes per trip as
// their 16-bit counterparts and cost the same per trip).  The 64 x 64
// tiles' trip costs were refitted after they went to three ring slots
// (256 x 4096 x 4096: 64 trips in 19.4 us; 512 x 512 x 16384 in 8 ranges).
//  - A launch costs kFixedUs plus the time to write C at kStoreBytesPerUs
//    (the outputs leave at the end of their tiles).
//  - Workgroups run in rounds of per_cu per CU.  A round that puts two on
//    some CU costs trip_shared per trip; a round of at most one per CU
//    costs trip_alone per trip, which for the 256 x 256 tiles grows with
//    the fraction of CUs busy (from trip_alone at none to trip_shared at
//    all: the chip runs at its power limit, so fewer busy CUs run faster).
//  - A split-K run adds its reduction, which moves every partial sum twice
//    (written by the GEMM, read back) at an effective kReduceBytesPerUs,
//    plus one launch.  The partial sums mostly stay in the last-level
//    cache: 2048 x 2048 x 16384 in four ranges measured 14 us of reduction.
struct TileCost {
  int per_cu;          // workgroups one CU runs at once
  double trip_alone;   // us per trip, at most one workgroup per CU
  double trip_shared;  // us per trip, two per CU (or every CU busy, per_cu = 1)
  bool power_scaled;   // trip_alone rises to trip_shared with the busy fraction
};
TileCost tile_cost(int id) {
  switch (id) {
    case 1: case 8: return {1, 0.93, 1.52, true};
    case 6: return {1, 0.56, 0.92, true};
    case 2: case 9: return {2, 0.75, 0.90, false};
    case 3: case 10: return {2, 0.26, 0.42, false};  // three slots in flight
    case 7: return {2, 0.31, 0.54, false};
    case 12: return {1, 0.65, 1.06, true};  // by rule (one round), by id and in the autotuner
    case 13: return {2, 0.38, 0.84, false};  // twice tile 3's work per trip
    default: return {1, 1.0, 1.0, false};  // 4, 5: chosen by rule or by id
  }
}
constexpr double kFixedUs = 3.0;
constexpr double kStoreBytesPerUs = 6.0e6;
constexpr double kReduceBytesPerUs = 10.0e6;
constexpr double kLaunchUs = 4.0;

double estimate_us(const gemm_desc& d, const gemm_device_caps& caps, int id, int64_t splits) {
  const auto& t = tile_desc(id);
  const TileCost c = tile_cost(id);
  const int64_t trips = std::max<int64_t>(cdiv(d.K, t.bk), 1);
  const int64_t tps = cdiv(trips, splits);
  const int64_t ranges = cdiv(trips, tps);
  const int64_t wgs = std::max<int64_t>(cdiv(d.M, t.bm) * cdiv(d.N, t.bn) * d.batch * ranges, 1);
  const int64_t cus = std::max(caps.num_cus, 1);
  const int64_t slots = cus * c.per_cu;
  const double mn = (double)d.M * (double)d.N * (double)d.batch;
  double us = kFixedUs + mn * out_size(d.out_dtype) / kStoreBytesPerUs;
  // Rounds of `slots` workgroups, then a last round of the rest; a round of
  // w workgroups costs tps trips at the price for w (closed form: the
  // number of rounds can be huge).
  auto trip_cost = [&](int64_t w) {
    if (w > cus) return c.trip_shared;
    if (c.power_scaled) return c.trip_alone + (c.trip_shared - c.trip_alone) * (double)w / (double)cus;
    return c.trip_alone;
  };
  const int64_t full = wgs / slots, rest = wgs % slots;
  us += (double)full * (double)tps * trip_cost(slots);
  if (rest > 0) us += (double)tps * trip_cost(rest);
  if (ranges > 1) us += (2.0 * ranges * mn * 4.0 + mn * out_size(d.out_dtype)) / kReduceBytesPerUs + kLaunchUs;
  return us;
}

// Problems the persistent short-K kernel (tile 11) takes: 16-bit operands,
// one batch item, 0 < K <= 96 and 0 < N <= 288 with 16-byte rows (K and N
// multiples of 8), no bias, the activation none or relu, staged, no split
// and no cap on the stage count.
bool shortk_fits(const gemm_desc& d) {
  using namespace tcg::shortk;
  return d.in_dtype != GEMM_FP8 && d.batch == 1 && d.M > 0 && d.K > 0 && d.K <= kKMax && d.K % 8 == 0 &&
         d.N > 0 && d.N <= kNMax && d.N % 8 == 0 && d.split_k <= 1 &&
         (d.epilogue == GEMM_EPI_NONE || d.epilogue == GEMM_EPI_RELU) &&
         !(d.flags & (GEMM_FLAG_BIAS | GEMM_FLAG_UNSTAGED | GEMM_FLAG_FORCE_STAGES_1 | GEMM_FLAG_FORCE_STAGES_2));
}

// Outputs the 256 x 128 tile (12) fills in one round of one workgroup per
// CU, without ragged tiles: 16-bit operands, one batch item, M a multiple of
// 256, N of 128, between 3/4 of the CUs and all of them busy.  Measured on
// MI355X (bf16, relu; 8192 x 1024, 4096 x 2048, 2048 x 4096 and 1024 x 8192,
// K 1024 to 4096): 0.7-10 % faster than the 128 x 128 tile the time model
// picks there, level at worst (+0.1 %).  Longer K is left to the model.
bool fills_one_round_256x128(const gemm_desc& d, const gemm_device_caps& caps) {
  if (d.in_dtype == GEMM_FP8 || d.batch != 1 || d.K <= 0 || d.K > 4096 || d.M <= 0 || d.N <= 0) return false;
  if (d.M % 256 || d.N % 128) return false;
  const int64_t grid = (d.M / 256) * (d.N / 128);
  return 4 * grid > 3 * (int64_t)caps.num_cus && grid <= (int64_t)caps.num_cus;
}

// Split counts the planner considers: powers of two while every range keeps
// at least kMinTripsPerSplit trips.
constexpr int64_t kMinTripsPerSplit = 8;

// Choose a tile (and, where allowed, a split) for the problem: short-K
// products whose N is a multiple of 96 take the 256 x 96 tile (few trips,
// many workgroups to stream A and C; measured faster than one 128 x 288 tile
// per row block); the rest take the tile and split with the lowest
// estimated time among 256 x 256, 128 x 128, 64 x 64, the 128 x 128
// ring of half-depth slots (which wins mid sizes such as 2048^3) and the
// 64 x 64 tile with 128-deep trips (half the trips, each with twice the
// MFMAs: it wins grids of at most one workgroup per CU without ragged
// tiles, 512^3 to 1024^3).
// Outputs that the 256 x 128 tile fills in exactly one round take it
// (fills_one_round_256x128).  Tiles 4-6 and 12 otherwise run only when asked
// for by id.  FP8 operands choose among
// their own tiles (8, 9, 10).
void choose(const gemm_desc& d, const gemm_device_caps& caps, bool may_split, int* tile, int64_t* splits) {
  *splits = 1;
  const bool fp8 = d.in_dtype == GEMM_FP8;
  if (d.tile) {
    *tile = d.tile;
    if (!may_split) return;
  } else if (shortk_fits(d) && d.M >= 2 * (int64_t)tcg::shortk::kBM * caps.num_cus) {
    // at least two blocks per workgroup, so that copies of later blocks
    // overlap the products and stores of earlier ones (at one to two
    // blocks, 40000 x 288 x 96, the 256 x 96 tile was level with it)
    *tile = 11;
    return;
  } else if (!fp8 && d.K <= 128 && d.N > 0 && d.N % 96 == 0) {
    *tile = 4;
    return;
  } else if (fills_one_round_256x128(d, caps)) {
    *tile = 12;
    return;
  }
  double best_t = 1e300;
  static const int kGeneral16[] = {1, 2, 3, 7, 13}, kGeneral8[] = {8, 9, 10};
  const int* ids = fp8 ? kGeneral8 : kGeneral16;
  int n_ids = fp8 ? 3 : 5;
  if (d.tile) {
    ids = &d.tile;
    n_ids = 1;
  }
  for (int k = 0; k < n_ids; ++k) {
    const int id = ids[k];
    const auto& t = tile_desc(id);
    const int64_t trips = cdiv(d.K, t.bk);
    const int64_t grid = cdiv(d.M, t.bm) * cdiv(d.N, t.bn) * d.batch;
    for (int64_t sp = 1; sp <= kMaxSplits; sp *= 2) {
      if (sp > 1 && (!may_split || trips / sp < kMinTripsPerSplit)) break;
      // The 128-deep 64 x 64 tile only where each CU runs at most one
      // workgroup (1536^3, 2.25 per CU: 20.5 us against 17.9 for the
      // 128 x 128 ring) and no tile is ragged (1000^3: 7.55 us against 7.45
      // for the 64-deep tile; 1024^3: 6.65 against 7.17).
      if (id == 13 && !d.tile && (grid * sp > caps.num_cus || d.M % t.bm || d.N % t.bn)) continue;
      const double est = estimate_us(d, caps, id, sp);
      if (est < best_t * 0.999) {
        best_t = est;
        *tile = id;
        *splits = sp;
      }
    }
  }
}

// A small last round of tiles: the rows of C whose tiles fill whole rounds
// run unsplit, and the rest as a second launch whose K is split so that it
// occupies more CUs.  Taken where the time model estimates it at least 3 %
// faster than one launch; the model's figures tracked measured ones on the
// 256 x 256 tile (bf16, one machine; one launch against head + split tail):
// 6144^3 402 against 370 us (tail 768 rows in 3 ranges), 4608^3 191 against
// 171, 7168^3 630 against 558 (256 rows in 8), while 5120^3 (a last round
// of 144 of 256 tiles) and 5120 x 5120 x 2048 lose, as estimated.
constexpr int kMaxTailSplit = 8;

bool tail_choice(const gemm_desc& d, const gemm_device_caps& caps, int id, int64_t* head_m, int* split) {
  const auto& t = tile_desc(id);
  if (t.persistent || d.batch != 1 || d.M <= 0 || d.N <= 0 || d.K <= 0) return false;
  const int64_t tiles_n = cdiv(d.N, t.bn), tiles = cdiv(d.M, t.bm) * tiles_n;
  const int64_t slots = (int64_t)caps.num_cus * tile_cost(id).per_cu;
  if (tiles <= slots || tiles % slots == 0) return false;
  // whole tile rows inside the whole rounds
  const int64_t rows = (tiles / slots) * slots / tiles_n;
  if (rows <= 0 || rows * t.bm >= d.M) return false;
  gemm_desc h = d, r = d;
  h.M = rows * t.bm;
  r.M = d.M - h.M;
  const double whole = estimate_us(d, caps, id, 1);
  const double head = estimate_us(h, caps, id, 1);
  const int64_t trips = cdiv(d.K, t.bk);
  double best = 1e300;
  for (int sp = 2; sp <= kMaxTailSplit && trips / sp >= kMinTripsPerSplit; ++sp) {
    const double e = head + estimate_us(r, caps, id, sp);
    if (e < best) {
      best = e;
      *split = sp;
    }
  }
  if (!(best < 0.97 * whole)) return false;
  *head_m = h.M;
  return true;
}

// ---------------------------------------------------------------------------
// Autotune cache: problem -> measured (tile, split).  The key is the
// device's architecture and CU count and every field of the normalised
// description but tile, split_k and GEMM_FLAG_TUNED.
// A measured choice: a tile and a split of K into `split` ranges, or
// split == 0 for the planner's own plan with its split tail (tile then
// names the tile that plan runs).
struct TuneChoice {
  int32_t tile;
  int32_t split;
  double us;
};
std::mutex g_tune_mu;
std::map<std::string, TuneChoice> g_tune;

std::string tune_key(const gemm_desc& d, const gemm_device_caps& caps) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s %d %lld %lld %lld %d %d %d %d %lld %lld %lld %lld", caps.arch, caps.num_cus,
                (long long)d.M, (long long)d.N, (long long)d.K, d.in_dtype, d.out_dtype, d.epilogue,
                d.flags & ~GEMM_FLAG_TUNED, (long long)d.batch, (long long)d.stride_a, (long long)d.stride_b,
                (long long)d.stride_c);
  return buf;
}

gemm_desc normalised(const gemm_desc& in) {
  gemm_desc d = in;
  if (d.batch == 1) {
    d.stride_a = d.M * d.K;
    d.stride_b = d.K * d.N;
    d.stride_c = d.M * d.N;
  }
  return d;
}

bool tuned_choice(const gemm_desc& d, const gemm_device_caps& caps, TuneChoice* out) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  auto it = g_tune.find(tune_key(d, caps));
  if (it == g_tune.end()) return false;
  *out = it->second;
  return true;
}

}  // namespace

// ---------------------------------------------------------------------------
extern "C" const char* gemm_strerror(int code) {
  switch (code) {
    case GEMM_OK: return "success";
    case GEMM_E_ARG: return "invalid argument (size, stride, flag, tile id or null pointer)";
    case GEMM_E_DTYPE: return "unsupported storage type (inputs: F16, BF16 or FP8 E4M3; output: F32, F16 or BF16)";
    case GEMM_E_ALIGN: return "pointer not aligned to its element size";
    case GEMM_E_ALIAS: return "C overlaps A or B (written parameters may not overlap others)";
    case GEMM_E_DEVICE: return "no usable gfx950 device, or the plan needs more LDS than it has";
    case GEMM_E_LAUNCH: return "kernel launch failed";
    case GEMM_E_NOMEM: return "host allocation failed";
    case GEMM_E_PLAN: return "null or destroyed plan";
    case GEMM_E_SIZE: return "problem too large: a tile's byte offsets exceed 31 bits";
    case GEMM_E_WORKSPACE: return "the plan splits K and needs a larger or 256-byte aligned workspace";
    case GEMM_E_SCRATCH: return "the plan needs a larger workspace than gemm_run_noalloc's fixed 64 MiB array";
    default: return "unknown error code";
  }
}

extern "C" int gemm_runtime_version(void) {
  int v = 0;
  if (hipRuntimeGetVersion(&v) != hipSuccess) return -1;
  return v;
}

extern "C" int gemm_tile_count(void) { return tcg::kNumTiles; }

extern "C" int gemm_device_caps_query(int device, gemm_device_caps* out) {
  if (!out) return GEMM_E_ARG;
  std::memset(out, 0, sizeof(*out));
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) {
    (void)hipGetLastError();
    return GEMM_E_DEVICE;
  }
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, device) != hipSuccess) return GEMM_E_DEVICE;
  out->num_cus = p.multiProcessorCount;
  out->wave_size = p.warpSize;
  out->clock_khz = p.clockRate;
  std::snprintf(out->arch, sizeof(out->arch), "%s", p.gcnArchName);
  int lds_block = 0, lds_optin = 0;
  (void)hipDeviceGetAttribute(&lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, device);
  (void)hipDeviceGetAttribute(&lds_optin, hipDeviceAttributeSharedMemPerBlockOptin, device);
  (void)hipGetLastError();
  out->lds_bytes = std::max<int>({lds_block, lds_optin, (int)p.sharedMemPerBlock});
  const bool gfx950 = std::strncmp(out->arch, "gfx950", 6) == 0;
  // gfx950 loads global memory straight into LDS without passing through
  // registers, so a copy overlaps the MFMAs that read the other slot.
  out->async_copy = gfx950 ? 1 : 0;
  out->num_xcds = gfx950 ? 8 : 1;
  if (log_enabled())
    std::fprintf(stderr, "[tcgemm] device %d: %s, %d CUs, LDS/workgroup %d (block %d, optin %d), clock %d kHz\n",
                 device, out->arch, out->num_cus, out->lds_bytes, lds_block, lds_optin, out->clock_khz);
  return gfx950 ? GEMM_OK : GEMM_E_DEVICE;
}

extern "C" int gemm_stage_depth(const gemm_device_caps* caps, int64_t used, const int64_t* tile_bytes,
                                int n_tiles, int stage_enabled) {
  if (!caps || !stage_enabled || n_tiles <= 0 || !tile_bytes) return 0;
  if (caps->lds_bytes <= 0 || caps->wave_size <= 0) return 0;
  int64_t sum = 0;
  for (int i = 0; i < n_tiles; ++i) {
    if (tile_bytes[i] < 16) return 0;  // less than one 16-byte copy
    sum += tile_bytes[i];
  }
  const int64_t avail = (int64_t)caps->lds_bytes - std::max<int64_t>(used, 0);
  if (caps->async_copy && 2 * sum <= avail) return 2;
  if (sum <= avail) return 1;
  return 0;
}

// The plan of the persistent short-K kernel.  It reports the 32-deep trips
// of the MFMA sequence it shares with tile 5 (bk = 32), so that a run whose
// pointers are not 16-byte aligned can take tile 5's kernel instead.
static int plan_shortk(const gemm_desc& d, const gemm_device_caps& caps, gemm_plan_t* out) {
  using namespace tcg::shortk;
  if (!shortk_fits(d)) return GEMM_E_ARG;
  if (caps.lds_bytes < kLdsBytes) return GEMM_E_DEVICE;
  const int64_t blocks = cdiv(d.M, kBM);
  if (blocks >= ((int64_t)1 << 30)) return GEMM_E_SIZE;
  Plan* p = new (std::nothrow) Plan();
  if (!p) return GEMM_E_NOMEM;
  p->magic = kPlanMagic;
  p->d = d;
  gemm_plan_info& in = p->info;
  in.tile_id = 11;
  in.bm = kBM;
  in.bn = kNMax;
  in.bk = 32;
  in.waves = 4;
  in.stages = kSlots;
  in.lds_bytes = kLdsBytes;
  in.vec16 = 1;
  in.tiles_m = blocks;
  in.tiles_n = 1;
  in.workgroups = std::min<int64_t>(blocks, std::max(caps.num_cus, 1));
  in.trips = cdiv(d.K, 32);
  in.mfma_per_run = blocks * 4 * kFN * 2 * in.trips;
  in.mfma_m = tcg::kMfmaM;
  in.mfma_n = tcg::kMfmaN;
  in.mfma_k = tcg::kMfmaK;
  in.split_k = 1;
  in.trips_per_split = in.trips;
  in.workspace_bytes = 0;
  p->group_m = (int32_t)std::min<int64_t>(4, blocks);
  p->xcd_remap = 0;
  std::snprintf(p->text, sizeof(p->text),
                "tile 11 (persistent, 128-row blocks, N <= %d, K <= %d, 4 waves), B image in LDS, %d A slots, "
                "LDS %d B, grid %lld over %lld blocks, trips %lld, mfma 32x32x16 %s, %lld MFMAs, epilogue %s",
                kNMax, kKMax, kSlots, kLdsBytes, (long long)in.workgroups, (long long)blocks, (long long)in.trips,
                d.in_dtype == GEMM_BF16 ? "bf16" : "f16", (long long)in.mfma_per_run,
                d.epilogue == GEMM_EPI_RELU ? "relu" : "none");
  if (log_enabled()) std::fprintf(stderr, "[tcgemm] plan %lldx%lldx%lld: %s\n", (long long)d.M,
                                  (long long)d.N, (long long)d.K, p->text);
  *out = reinterpret_cast<gemm_plan_t>(p);
  return GEMM_OK;
}

// The plan of a problem whose last rows run with K split (tail_choice): two
// sub-plans of the same tile, made by id.
int plan_with_tail(const gemm_desc& d, const gemm_device_caps& caps, int id, int64_t head_m, int split,
                   gemm_plan_t* out) {
  gemm_desc h = d, r = d;
  h.flags &= ~(GEMM_FLAG_SPLIT_K | GEMM_FLAG_TUNED);
  r.flags = h.flags;
  h.tile = r.tile = id;
  h.M = head_m;
  h.split_k = 1;
  r.M = d.M - head_m;
  r.split_k = split;
  gemm_plan_t hp = nullptr, rp = nullptr;
  int rc = gemm_plan_for_caps(&h, &caps, &hp);
  if (rc == GEMM_OK) rc = gemm_plan_for_caps(&r, &caps, &rp);
  Plan* p = rc == GEMM_OK ? new (std::nothrow) Plan() : nullptr;
  if (!p) {
    gemm_plan_destroy(hp);
    gemm_plan_destroy(rp);
    return rc != GEMM_OK ? rc : GEMM_E_NOMEM;
  }
  Plan* H = reinterpret_cast<Plan*>(hp);
  Plan* R = reinterpret_cast<Plan*>(rp);
  p->magic = kPlanMagic;
  p->d = d;
  p->info = H->info;
  p->group_m = H->group_m;
  p->xcd_remap = H->xcd_remap;
  p->head = H;
  p->tail = R;
  gemm_plan_info& in = p->info;
  in.workgroups += R->info.workgroups;
  in.mfma_per_run += R->info.mfma_per_run;
  in.workspace_bytes = R->info.workspace_bytes;
  in.tail_rows = r.M;
  in.tail_split = R->info.split_k;
  std::snprintf(p->text, sizeof(p->text), "%s; last %lld rows a second launch, split K %d x %lld trips (%lld workgroups, workspace %lld B)",
                H->text, (long long)r.M, R->info.split_k, (long long)R->info.trips_per_split,
                (long long)R->info.workgroups, (long long)R->info.workspace_bytes);
  if (log_enabled()) std::fprintf(stderr, "[tcgemm] plan %lldx%lldx%lld: %s\n", (long long)d.M,
                                  (long long)d.N, (long long)d.K, p->text);
  *out = reinterpret_cast<gemm_plan_t>(p);
  return GEMM_OK;
}

extern "C" int gemm_plan_for_caps(const gemm_desc* desc, const gemm_device_caps* caps, gemm_plan_t* out) {
  if (!out) return GEMM_E_ARG;
  *out = nullptr;
  int rc = validate_desc(desc);
  if (rc) return rc;
  if (!caps || caps->num_cus <= 0 || caps->wave_size != 64) return GEMM_E_DEVICE;
  gemm_desc d = normalised(*desc);
  TuneChoice tc;
  if ((d.flags & GEMM_FLAG_TUNED) && d.tile == 0 && d.split_k == 0 && tuned_choice(d, *caps, &tc) &&
      tc.split > 0) {
    d.tile = tc.tile;
    d.split_k = tc.split;
  }  // (split 0: the planner's own plan with a split tail won; plan it again below)
  int id = 0;
  int64_t want_splits = 1;
  if (d.split_k > 0) {
    choose(d, *caps, false, &id, &want_splits);
    want_splits = d.split_k;
  } else {
    choose(d, *caps, (d.flags & GEMM_FLAG_SPLIT_K) != 0, &id, &want_splits);
  }
  const auto& t = tile_desc(id);
  if (t.persistent) return plan_shortk(d, *caps, out);
  int64_t head_m = 0;
  int tail_split = 0;
  if (d.tile == 0 && d.split_k == 0 && (d.flags & GEMM_FLAG_SPLIT_K) && want_splits == 1 &&
      tail_choice(d, *caps, id, &head_m, &tail_split))
    return plan_with_tail(d, *caps, id, head_m, tail_split, out);

  const int64_t tiles[2] = {(int64_t)t.bm * t.bk * t.esize, (int64_t)t.bk * t.bn * t.esize};
  int stages = gemm_stage_depth(caps, 0, tiles, 2, (d.flags & GEMM_FLAG_UNSTAGED) ? 0 : 1);
  // Where two stages fit and the tile's kernel is built for a deeper ring,
  // keep more chunks in flight while they fit: more stages hide longer
  // memory latency at the cost of LDS (page "gizml:tile", Program.stages).
  // With 4 trips or fewer a deeper ring only delays the first products
  // (measured on the 64 x 64 tile: 256^3, 4 trips, 3.7 us with two slots
  // and 4.0 us with three).
  // A deeper ring that leaves room for fewer workgroups per CU than the
  // tile is built for (the 64 x 64 x 128 tile: three 32 KiB slots) pays
  // only while the grid runs in one round and K is long: measured on that
  // tile, 1024^3 (8 trips) 6.7 us with two slots and 7.1 with three,
  // 512 x 512 x 8192 39.2 and 26.9 us, 2048^3 (four workgroups per CU)
  // 31.2 and 36.0 us.
  if (stages == 2 && t.max_stages > 2 && !(d.flags & GEMM_FLAG_FORCE_STAGES_2) && cdiv(d.K, t.bk) > 4) {
    const int64_t fit = (int64_t)caps->lds_bytes / (tiles[0] + tiles[1]);
    int deeper = (int)std::min<int64_t>(t.max_stages, fit);
    const bool fewer_per_cu = (int64_t)t.min_waves * tcg::lds_bytes_for(t, deeper) > caps->lds_bytes;
    const int64_t sp = std::max<int64_t>(want_splits, 1);
    const int64_t grid = cdiv(d.M, t.bm) * cdiv(d.N, t.bn) * std::max<int64_t>(d.batch, 1) * sp;
    if (fewer_per_cu && (cdiv(cdiv(d.K, t.bk), sp) <= 8 || grid > caps->num_cus)) deeper = 2;
    stages = deeper;
  }
  if ((d.flags & GEMM_FLAG_FORCE_STAGES_1) && stages > 1) stages = 1;

  // The first slot also holds the epilogue bands, which can be larger than
  // a slot for small tiles; even the unstaged kernel needs the bands.
  while (stages > 0 && tcg::lds_bytes_for(t, stages) > caps->lds_bytes) --stages;
  if (tcg::lds_bytes_for(t, stages) > caps->lds_bytes) return GEMM_E_DEVICE;
  // Byte offsets inside one trip's tiles are 32-bit buffer offsets.
  if ((int64_t)t.bm * std::max<int64_t>(d.K, 1) * t.esize >= (int64_t)0x7fffffff ||
      (int64_t)t.bk * std::max<int64_t>(d.N, 1) * t.esize >= (int64_t)0x7fffffff)
    return GEMM_E_SIZE;
  const int64_t tiles_m = cdiv(d.M, t.bm), tiles_n = cdiv(d.N, t.bn);
  const int64_t trips = cdiv(d.K, t.bk);
  // K ranges of whole trips; none empty (K == 0 keeps one range).
  const bool can_split = trips > 0 && d.M > 0 && d.N > 0;
  const int64_t tps = can_split ? cdiv(trips, std::min<int64_t>(want_splits, trips)) : trips;
  const int64_t splits = can_split ? cdiv(trips, tps) : 1;
  const int64_t wgs = tiles_m * tiles_n * d.batch * splits;
  const int nt = t.wm * t.wn * 64;
  if (wgs * nt >= ((int64_t)1 << 32) || trips > 0x7fffffff) return GEMM_E_SIZE;
  const int64_t ws_bytes = splits > 1 ? splits * d.batch * d.M * d.N * 4 : 0;

  Plan* p = new (std::nothrow) Plan();
  if (!p) return GEMM_E_NOMEM;
  p->magic = kPlanMagic;
  p->d = d;
  gemm_plan_info& in = p->info;
  in.tile_id = id;
  in.bm = t.bm;
  in.bn = t.bn;
  in.bk = t.bk;
  in.waves = t.wm * t.wn;
  in.stages = stages;
  in.lds_bytes = tcg::lds_bytes_for(t, stages);
  const int64_t epc = 16 / t.esize;  // elements per 16-byte copy
  in.vec16 = (d.K % epc == 0 && d.N % epc == 0 && d.stride_a % epc == 0 && d.stride_b % epc == 0) ? 1 : 0;
  in.tiles_m = tiles_m;
  in.tiles_n = tiles_n;
  in.workgroups = wgs;
  in.trips = trips;
  const int fm = t.bm / t.wm / tcg::kMfmaM, fn = t.bn / t.wn / tcg::kMfmaN;
  in.mfma_per_run = tiles_m * tiles_n * d.batch * in.waves * fm * fn * in.trips * (t.bk / tcg::mfma_k(t));
  in.mfma_m = tcg::kMfmaM;
  in.mfma_n = tcg::kMfmaN;
  in.mfma_k = tcg::mfma_k(t);
  in.split_k = (int32_t)splits;
  in.trips_per_split = tps;
  in.workspace_bytes = ws_bytes;
  p->group_m = (int32_t)std::max<int64_t>(1, std::min<int64_t>(4, tiles_m));
  p->xcd_remap = caps->num_xcds == 8 ? 1 : 0;
  static const char* const kActName[] = {"none", "relu", "gelu", "gelu_erf", "sigmoid", "tanh"};
  char split_text[96] = "";
  if (splits > 1)
    std::snprintf(split_text, sizeof(split_text), ", split K %lld x %lld trips (workspace %lld B)",
                  (long long)splits, (long long)tps, (long long)ws_bytes);
  std::snprintf(p->text, sizeof(p->text),
                "tile %d (%dx%dx%d, %d waves), stages %d, LDS %d B, %s copies, grid %lld (%lldx%lld x %lld%s), "
                "trips %lld, mfma %dx%dx%d %s, %lld MFMAs, epilogue %s%s%s",
                id, t.bm, t.bn, t.bk, in.waves, stages, in.lds_bytes, in.vec16 ? "16-byte" : "element",
                (long long)wgs, (long long)tiles_m, (long long)tiles_n, (long long)d.batch,
                splits > 1 ? " x splits" : "", (long long)in.trips, in.mfma_m, in.mfma_n, in.mfma_k,
                d.in_dtype == GEMM_BF16 ? "bf16" : (d.in_dtype == GEMM_FP8 ? "fp8" : "f16"),
                (long long)in.mfma_per_run,
                (d.flags & GEMM_FLAG_BIAS) ? "bias+" : "", kActName[d.epilogue], split_text);
  if (log_enabled()) std::fprintf(stderr, "[tcgemm] plan %lldx%lldx%lld: %s\n", (long long)d.M,
                                  (long long)d.N, (long long)d.K, p->text);
  *out = reinterpret_cast<gemm_plan_t>(p);
  return GEMM_OK;
}

extern "C" int gemm_plan(const gemm_desc* desc, gemm_plan_t* out) {
  if (!out) return GEMM_E_ARG;
  *out = nullptr;
  int rc = validate_desc(desc);
  if (rc) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_E_DEVICE;
  }
  gemm_device_caps caps;
  rc = cached_caps(dev, &caps);
  if (rc) return rc;
  return gemm_plan_for_caps(desc, &caps, out);
}

static Plan* as_plan(gemm_plan_t h) {
  Plan* p = reinterpret_cast<Plan*>(h);
  return (p && p->magic == kPlanMagic) ? p : nullptr;
}

extern "C" int gemm_plan_get_info(gemm_plan_t plan, gemm_plan_info* out) {
  Plan* p = as_plan(plan);
  if (!p) return GEMM_E_PLAN;
  if (!out) return GEMM_E_ARG;
  *out = p->info;
  return GEMM_OK;
}

extern "C" const char* gemm_plan_describe(gemm_plan_t plan) {
  Plan* p = as_plan(plan);
  return p ? p->text : "(invalid plan)";
}

extern "C" void gemm_plan_destroy(gemm_plan_t plan) {
  Plan* p = as_plan(plan);
  if (!p) return;
  p->magic = 0;
  if (p->head) gemm_plan_destroy(reinterpret_cast<gemm_plan_t>(p->head));
  if (p->tail) gemm_plan_destroy(reinterpret_cast<gemm_plan_t>(p->tail));
  delete p;
}

static bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) {
  return a0 < b1 && b0 < a1;
}

extern "C" int gemm_run(gemm_plan_t plan, const void* A, const void* B, void* C, void* stream) {
  return gemm_run_ex(plan, A, B, C, nullptr, stream);
}

extern "C" int gemm_run_ex(gemm_plan_t plan, const void* A, const void* B, void* C, const gemm_run_args* args,
                           void* stream) {
  Plan* p = as_plan(plan);
  if (!p) return GEMM_E_PLAN;
  const gemm_desc& d = p->d;
  const gemm_plan_info& in = p->info;
  if (args && (args->reserved[0] | args->reserved[1] | args->reserved[2] | args->reserved[3]))
    return GEMM_E_ARG;
  const bool want_bias = (d.flags & GEMM_FLAG_BIAS) != 0;
  const float* bias = want_bias && args ? static_cast<const float*>(args->bias) : nullptr;
  if (want_bias && !bias) return GEMM_E_ARG;
  if (bias && ((uintptr_t)bias & 3u)) return GEMM_E_ALIGN;
  float* ws = nullptr;
  if (in.split_k > 1 || in.tail_rows > 0) {
    if (!args || !args->workspace || args->workspace_bytes < in.workspace_bytes ||
        ((uintptr_t)args->workspace & 255u))
      return GEMM_E_WORKSPACE;
    ws = static_cast<float*>(args->workspace);
  }
  if (d.M == 0 || d.N == 0) return GEMM_OK;
  if (!C || (d.K > 0 && (!A || !B))) return GEMM_E_ARG;
  const int osz = out_size(d.out_dtype);
  const int isz = in_size(d.in_dtype);
  if (((uintptr_t)A & (uintptr_t)(isz - 1)) || ((uintptr_t)B & (uintptr_t)(isz - 1)) ||
      ((uintptr_t)C & (uintptr_t)(osz - 1)))
    return GEMM_E_ALIGN;
  // Written parameters may not overlap the others (page "Module Tolk.Uniform", precondition).
  const uintptr_t c0 = (uintptr_t)C;
  const uintptr_t c1 = c0 + (uintptr_t)(((d.batch - 1) * d.stride_c + d.M * d.N) * osz);
  if (d.K > 0) {
    const uintptr_t a0 = (uintptr_t)A, a1 = a0 + (uintptr_t)(((d.batch - 1) * d.stride_a + d.M * d.K) * isz);
    const uintptr_t b0 = (uintptr_t)B, b1 = b0 + (uintptr_t)(((d.batch - 1) * d.stride_b + d.K * d.N) * isz);
    if (overlaps(c0, c1, a0, a1) || overlaps(c0, c1, b0, b1)) return GEMM_E_ALIAS;
    if (ws) {
      const uintptr_t w0 = (uintptr_t)ws, w1 = w0 + (uintptr_t)in.workspace_bytes;
      if (overlaps(w0, w1, a0, a1) || overlaps(w0, w1, b0, b1)) return GEMM_E_ALIAS;
    }
  }
  if (bias) {
    const uintptr_t z0 = (uintptr_t)bias, z1 = z0 + (uintptr_t)(d.N * 4);
    if (overlaps(z0, z1, c0, c1)) return GEMM_E_ALIAS;
    if (ws && overlaps(z0, z1, (uintptr_t)ws, (uintptr_t)ws + (uintptr_t)in.workspace_bytes)) return GEMM_E_ALIAS;
  }
  if (ws && overlaps((uintptr_t)ws, (uintptr_t)ws + (uintptr_t)in.workspace_bytes, c0, c1)) return GEMM_E_ALIAS;
  if (p->tail) {
    // the rows above the tail, then the tail rows (same stream, in order)
    const int64_t hm = p->head->d.M;
    const int rc = gemm_run_ex(reinterpret_cast<gemm_plan_t>(p->head), A, B, C, args, stream);
    if (rc != GEMM_OK) return rc;
    return gemm_run_ex(reinterpret_cast<gemm_plan_t>(p->tail), static_cast<const char*>(A) + hm * d.K * isz, B,
                       static_cast<char*>(C) + hm * d.N * osz, args, stream);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_E_DEVICE;
  }
  gemm_device_caps caps;
  if (cached_caps(dev, &caps) != GEMM_OK || !is_gfx950(caps) || caps.lds_bytes < in.lds_bytes)
    return GEMM_E_DEVICE;

  tcg::KArgs a;
  a.A = A;
  a.B = B;
  a.C = C;
  a.bias = bias;
  a.ws = ws;
  a.M = d.M;
  a.N = d.N;
  a.K = d.K;
  a.stride_a = d.stride_a;
  a.stride_b = d.stride_b;
  a.stride_c = d.stride_c;
  a.tiles_m = in.tiles_m;
  a.tiles_n = in.tiles_n;
  a.batch = d.batch;
  a.workgroups = in.workgroups;
  a.trips = (int32_t)in.trips;
  a.splits = in.split_k;
  a.trips_per_split = (int32_t)in.trips_per_split;
  a.out_dtype = d.out_dtype;
  a.act = d.epilogue;
  a.ws_vec = d.N % 4 == 0 ? 1 : 0;
  a.group_m = p->group_m;
  a.xcd_remap = p->xcd_remap;
  a.vec_store4 = (d.N % 4 == 0 && (c0 % (uintptr_t)(4 * osz)) == 0 && (d.batch == 1 || d.stride_c % 4 == 0)) ? 1 : 0;
  const int64_t per16 = 16 / osz;
  a.vec_store16 = (d.N % per16 == 0 && (c0 % 16u) == 0 && (d.batch == 1 || d.stride_c % per16 == 0)) ? 1 : 0;
  const bool vec16 = in.vec16 && ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0);
  const bool bf16 = d.in_dtype == GEMM_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipErrorInvalidValue;
  // The general epilogue's kernels only where the GEMM finishes C itself
  // with a bias or a transcendental activation.
  const bool gen = in.split_k == 1 && (bias || (d.epilogue != GEMM_EPI_NONE && d.epilogue != GEMM_EPI_RELU));
  if (in.tile_id == 11) {
    if (vec16 && a.vec_store16 && (c0 % 16u) == 0) {
      e = tcg::launch_t11(bf16, a, s);
    } else {
      // Rows not 16-byte aligned: tile 5's kernel, the same MFMA sequence
      // (identical bits), with element copies or element stores.
      a.workgroups = in.tiles_m;
      a.group_m = (int32_t)std::min<int64_t>(4, in.tiles_m);
      e = tcg::launch_t5(2, vec16, bf16, a, s);
    }
  }
  switch (in.tile_id) {
    case 1: e = (gen ? tcg::launch_t1_gen : tcg::launch_t1)(in.stages, vec16, bf16, a, s); break;
    case 2: e = (gen ? tcg::launch_t2_gen : tcg::launch_t2)(in.stages, vec16, bf16, a, s); break;
    case 3: e = (gen ? tcg::launch_t3_gen : tcg::launch_t3)(in.stages, vec16, bf16, a, s); break;
    case 4: e = (gen ? tcg::launch_t4_gen : tcg::launch_t4)(in.stages, vec16, bf16, a, s); break;
    case 5: e = (gen ? tcg::launch_t5_gen : tcg::launch_t5)(in.stages, vec16, bf16, a, s); break;
    case 6: e = (gen ? tcg::launch_t6_gen : tcg::launch_t6)(in.stages, vec16, bf16, a, s); break;
    case 7: e = (gen ? tcg::launch_t7_gen : tcg::launch_t7)(in.stages, vec16, bf16, a, s); break;
    case 8: e = (gen ? tcg::launch_t8_gen : tcg::launch_t8)(in.stages, vec16, bf16, a, s); break;
    case 9: e = (gen ? tcg::launch_t9_gen : tcg::launch_t9)(in.stages, vec16, bf16, a, s); break;
    case 10: e = (gen ? tcg::launch_t10_gen : tcg::launch_t10)(in.stages, vec16, bf16, a, s); break;
    case 12: e = (gen ? tcg::launch_t12_gen : tcg::launch_t12)(in.stages, vec16, bf16, a, s); break;
    case 13: e = (gen ? tcg::launch_t13_gen : tcg::launch_t13)(in.stages, vec16, bf16, a, s); break;
    default: break;
  }
  if (e == hipSuccess && in.split_k > 1) {
    tcg::RArgs r;
    r.ws = ws;
    r.C = C;
    r.bias = bias;
    r.M = d.M;
    r.N = d.N;
    r.batch = d.batch;
    r.stride_c = d.stride_c;
    r.splits = in.split_k;
    r.out_dtype = d.out_dtype;
    r.act = d.epilogue;
    r.vec4 = a.vec_store4;
    e = tcg::launch_splitk_reduce(r, s);
  }
  if (e != hipSuccess) {
    if (log_enabled()) std::fprintf(stderr, "[tcgemm] launch failed: %s\n", hipGetErrorString(e));
    return GEMM_E_LAUNCH;
  }
  return GEMM_OK;
}

// ---------------------------------------------------------------------------
// Autotune (page "gizml:tile", tune).
extern "C" int gemm_autotune(const gemm_desc* desc, const void* A, const void* B, void* C,
                             const gemm_run_args* args, void* stream, gemm_plan_t* out) {
  if (!out) return GEMM_E_ARG;
  *out = nullptr;
  int rc = validate_desc(desc);
  if (rc) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_E_DEVICE;
  }
  gemm_device_caps caps;
  rc = cached_caps(dev, &caps);
  if (rc) return rc;
  const gemm_desc base = normalised(*desc);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    (void)hipGetLastError();
    return GEMM_E_LAUNCH;
  }
  const int64_t ws_have = (args && args->workspace) ? args->workspace_bytes : 0;
  const int lo = base.tile ? base.tile : 1, hi = base.tile ? base.tile : tcg::kNumTiles;
  TuneChoice best{0, 1, 1e300};
  rc = GEMM_OK;
  // One warm-up run, then the fastest of five timed runs of plan h (us), or
  // an error code in *err.
  auto time_plan = [&](gemm_plan_t h, int* err) {
    double t_min = 1e300;
    int r = gemm_run_ex(h, A, B, C, args, stream);  // warm-up
    for (int rep = 0; rep < 5 && r == GEMM_OK; ++rep) {
      float ms = 0.0f;
      if (hipEventRecord(e0, s) != hipSuccess || (r = gemm_run_ex(h, A, B, C, args, stream)) != GEMM_OK ||
          hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
          hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
        if (r == GEMM_OK) r = GEMM_E_LAUNCH;
        break;
      }
      t_min = std::min(t_min, 1e3 * (double)ms);
    }
    *err = r;
    return t_min;
  };
  // A description that names a tile or a split restricts the search to it;
  // such a result answers only that question and is not cached.
  const bool restricted = base.tile != 0 || base.split_k != 0;
  for (int id = lo; id <= hi && rc == GEMM_OK; ++id) {
    if (tcg::kTiles[id - 1].esize != in_size(base.in_dtype)) continue;  // built for the other width
    int last_split = 0;
    const int sp_first = base.split_k > 0 ? base.split_k : 1;
    const int sp_last = base.split_k > 0 ? base.split_k : ((base.flags & GEMM_FLAG_SPLIT_K) ? 16 : 1);
    for (int sp = sp_first; sp <= sp_last; sp *= 2) {
      gemm_desc d = base;
      d.tile = id;
      d.split_k = sp;
      d.flags &= ~GEMM_FLAG_TUNED;
      gemm_plan_t h = nullptr;
      if (gemm_plan_for_caps(&d, &caps, &h) != GEMM_OK) continue;
      const gemm_plan_info& in = reinterpret_cast<Plan*>(h)->info;
      const bool usable = in.split_k == sp && in.split_k != last_split && in.workspace_bytes <= ws_have &&
                          (sp == 1 || base.split_k > 0 || in.trips_per_split >= 4);
      if (!usable) {
        gemm_plan_destroy(h);
        continue;
      }
      last_split = in.split_k;
      int r = GEMM_OK;
      const double t_min = time_plan(h, &r);
      gemm_plan_destroy(h);
      if (r != GEMM_OK) {
        rc = r;
        break;
      }
      if (log_enabled())
        std::fprintf(stderr, "[tcgemm] tune %lldx%lldx%lld: tile %d split %d: %.2f us\n", (long long)d.M,
                     (long long)d.N, (long long)d.K, id, sp, t_min);
      if (t_min < best.us) best = TuneChoice{id, sp, t_min};
    }
  }
  // The planner's own plan where it splits K for the bottom rows only (a
  // small last round of tiles): a candidate of its own, kept as split 0.
  if (rc == GEMM_OK && base.tile == 0 && base.split_k == 0 && (base.flags & GEMM_FLAG_SPLIT_K)) {
    gemm_desc d = base;
    d.flags &= ~GEMM_FLAG_TUNED;
    gemm_plan_t h = nullptr;
    if (gemm_plan_for_caps(&d, &caps, &h) == GEMM_OK) {
      const gemm_plan_info& in = reinterpret_cast<Plan*>(h)->info;
      if (in.tail_rows > 0 && in.workspace_bytes <= ws_have) {
        int r = GEMM_OK;
        const double t_min = time_plan(h, &r);
        if (r != GEMM_OK) rc = r;
        if (r == GEMM_OK && log_enabled())
          std::fprintf(stderr, "[tcgemm] tune %lldx%lldx%lld: planner's split tail (tile %d): %.2f us\n",
                       (long long)d.M, (long long)d.N, (long long)d.K, in.tile_id, t_min);
        if (r == GEMM_OK && t_min < best.us) best = TuneChoice{in.tile_id, 0, t_min};
      }
      gemm_plan_destroy(h);
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipGetLastError();
  if (rc != GEMM_OK) return rc;
  if (best.tile == 0) return GEMM_E_PLAN;  // no candidate could run
  if (!restricted) {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    g_tune[tune_key(base, caps)] = best;
  }
  gemm_desc d = base;
  if (best.split > 0) {
    d.tile = best.tile;
    d.split_k = best.split;
  }  // else the planner's own plan (its split tail)
  d.flags &= ~GEMM_FLAG_TUNED;
  return gemm_plan_for_caps(&d, &caps, out);
}

extern "C" int gemm_tune_cache_save(const char* path) {
  if (!path) return GEMM_E_ARG;
  FILE* f = std::fopen(path, "w");
  if (!f) return GEMM_E_ARG;
  std::lock_guard<std::mutex> lk(g_tune_mu);
  for (const auto& kv : g_tune)
    std::fprintf(f, "%s %d %d %.3f\n", kv.first.c_str(), kv.second.tile, kv.second.split, kv.second.us);
  return std::fclose(f) == 0 ? GEMM_OK : GEMM_E_ARG;
}

extern "C" int gemm_tune_cache_load(const char* path) {
  if (!path) return GEMM_E_ARG;
  FILE* f = std::fopen(path, "r");
  if (!f) return GEMM_E_ARG;
  char line[512];
  int rc = GEMM_OK;
  std::map<std::string, TuneChoice> read;
  while (std::fgets(line, sizeof(line), f)) {
    char arch[64];
    int cus, in, o, epi, flags, tile, split;
    long long M, N, K, batch, sa, sb, sc;
    double us;
    if (std::sscanf(line, "%63s %d %lld %lld %lld %d %d %d %d %lld %lld %lld %lld %d %d %lf", arch, &cus, &M, &N,
                    &K, &in, &o, &epi, &flags, &batch, &sa, &sb, &sc, &tile, &split, &us) != 16 ||
        tile < 1 || tile > tcg::kNumTiles || split < 0 || split > kMaxSplits) {
      rc = GEMM_E_ARG;
      break;
    }
    char key[256];
    std::snprintf(key, sizeof(key), "%s %d %lld %lld %lld %d %d %d %d %lld %lld %lld %lld", arch, cus, M, N, K, in,
                  o, epi, flags, batch, sa, sb, sc);
    read[key] = TuneChoice{tile, split, us};
  }
  std::fclose(f);
  if (rc != GEMM_OK) return rc;
  std::lock_guard<std::mutex> lk(g_tune_mu);
  for (const auto& kv : read) g_tune[kv.first] = kv.second;
  return GEMM_OK;
}

extern "C" void gemm_tune_cache_clear(void) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tune.clear();
}

extern "C" int gemm_tune_cache_size(void) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  return (int)g_tune.size();
}
