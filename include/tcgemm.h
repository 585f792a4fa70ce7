/*
 * tcgemm.h -- C ABI of libtcgemm.so: C = epilogue(A . B) on an AMD Instinct
 * MI355X (gfx950), with operand tiles staged through LDS before the MFMA
 * units read their fragments.
 *
 * What one run computes, for every batch item b, row i < M, column j < N
 * (page "gizml:tile": the worked example, Program.zeros, Program.fold,
 * Tile.dot, Tile.relu, Tile.to, In.at, Out.put):
 *
 *     acc = +0, then acc += A[b,i,k] * B[b,k,j] for k = 0 .. K-1, in fp32
 *     v   = bias ? acc + bias[j] : acc                    (Tile.add, broadcast)
 *     y   = act(v)   (none, relu, gelu, geluErf, sigmoid or tanh, in fp32)
 *     C[b,i,j] = y rounded to nearest-even in the output storage type
 *
 * With a split K (desc.split_k > 1, or GEMM_FLAG_SPLIT_K and the planner's
 * choice) the K range is cut into split_k consecutive ranges of whole trips;
 * each range's sum is formed as above and the ranges' sums are then added in
 * ascending order in fp32 before the epilogue.  This reassociates the fold:
 * the result is exact wherever every partial sum is exact (integer inputs
 * whose sums stay below 2^24) and otherwise differs from the unsplit fold by
 * rounding only.  Every path of one plan (staged, one stage, unstaged)
 * splits the same way and returns the same bits.
 *
 * With GEMM_FLAG_SPLIT_K the planner may also split K for the bottom rows
 * only (gemm_plan_info.tail_rows > 0): where the output tiles fill some
 * whole rounds of the device's CUs and leave a small last round, the rows
 * of the whole rounds run unsplit and the last tail_rows rows run as a
 * second launch (same stream) with K cut into tail_split ranges, so that
 * the last round occupies more CUs.  Rows above the tail return the
 * unsplit plan's bits; tail rows return the bits of a plan split into
 * tail_split ranges.
 *
 * Elements outside the matrices read as 0 (In.at) and elements outside C are
 * never written (Out.put leaves the rest of C as it was).  The staged kernel
 * and the unstaged kernel of the same plan perform the same MFMA sequence on
 * the same values, so they return the same bits (page "Module Tolk.Stage":
 * staging copies values unchanged).
 *
 * Layout: A is [batch][M][K], B is [batch][K][N], C is [batch][M][N], all
 * row-major with contiguous rows (row pitch K, N and N elements).  stride_*
 * is the distance in elements between consecutive batch items (ignored when
 * batch == 1).  Storage codes are the page's constants (F32 = 0, F16 = 4,
 * BF16 = 5); A and B share one input type (Tile.dot multiplies operands of the same type).
 *
 * Threading: plans are immutable after creation and may be used from any
 * thread and on any stream.  gemm_run allocates nothing, never
 * synchronises, and is asynchronous with respect to the host.
 *
 * Errors: every int-returning call returns GEMM_OK (0) or a negative
 * GEMM_E_* code; gemm_strerror names it.  (Named, specific failures follow
 * the error convention of the page "Module Tolk.Uniform", check.)
 */
#ifndef TCGEMM_H
#define TCGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage codes (page "gizml:tile", Constants).  FP8 is E4M3, read as the
 * OCP 8-bit format (bias 7, no infinities, NaN at S.1111.111, largest 448);
 * it is an operand type only (A and B), outputs are F32, F16 or BF16. */
enum { GEMM_F32 = 0, GEMM_F16 = 4, GEMM_BF16 = 5, GEMM_FP8 = 9 };

/* Activations applied after the optional bias (page "gizml:tile": Tile.relu,
 * Tile.gelu, Tile.geluErf, Tile.sigmoid, Tile.tanh):
 *   RELU      max(v, 0), with NaN and -0 giving +0
 *   GELU      the tanh form: v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))) / 2
 *   GELU_ERF  the erf form:  v (1 + erf(v / sqrt(2))) / 2
 *   SIGMOID   1 / (1 + e^-v)
 *   TANH      tanh(v)
 * The transcendental ones are evaluated in fp32 with the device math
 * library (a few ulp), then rounded to the output type. */
enum {
  GEMM_EPI_NONE = 0,
  GEMM_EPI_RELU = 1,
  GEMM_EPI_GELU = 2,
  GEMM_EPI_GELU_ERF = 3,
  GEMM_EPI_SIGMOID = 4,
  GEMM_EPI_TANH = 5
};

/* Plan flags.
 *   GEMM_FLAG_FORCE_STAGES_1: use at most one LDS stage even where two fit.
 *   GEMM_FLAG_UNSTAGED: no LDS staging; fragments are loaded straight from
 *     global memory (the "Setting.stage off" case of the page "Module
 *     Tolk.Stage", depth).
 *   GEMM_FLAG_FORCE_STAGES_2: use at most two stages even where the tile's
 *     kernel could keep more chunks in flight.
 *   GEMM_FLAG_BIAS: add a bias row before the activation: N fp32 values,
 *     bias[j] added to column j of every row of every batch item (passed
 *     to gemm_run_ex).
 *   GEMM_FLAG_SPLIT_K: with split_k == 0, let the planner split K where
 *     that is estimated faster (few output tiles, long K), or split it for
 *     the bottom rows only (a small last round of tiles, batch 1); such a
 *     plan needs a workspace (gemm_plan_info.workspace_bytes).
 *   GEMM_FLAG_TUNED: with tile == 0 and split_k == 0, take the choice an
 *     earlier gemm_autotune measured for this problem on this device, if
 *     any (else the planner's). */
enum {
  GEMM_FLAG_FORCE_STAGES_1 = 1,
  GEMM_FLAG_UNSTAGED = 2,
  GEMM_FLAG_FORCE_STAGES_2 = 4,
  GEMM_FLAG_BIAS = 8,
  GEMM_FLAG_SPLIT_K = 16,
  GEMM_FLAG_TUNED = 32
};

/* Error codes. */
enum {
  GEMM_OK = 0,
  GEMM_E_ARG = -1,     /* bad size, stride, flag, tile id or null pointer      */
  GEMM_E_DTYPE = -2,   /* unsupported input/output storage type                */
  GEMM_E_ALIGN = -3,   /* a pointer is not aligned to its element size         */
  GEMM_E_ALIAS = -4,   /* C overlaps A or B (page "Module Tolk.Uniform":
                          parameters that are written may not overlap others) */
  GEMM_E_DEVICE = -5,  /* no usable gfx950 device, or the plan does not fit it */
  GEMM_E_LAUNCH = -6,  /* the kernel launch failed (hipGetLastError)           */
  GEMM_E_NOMEM = -7,   /* host allocation of the plan failed                   */
  GEMM_E_PLAN = -8,    /* null or destroyed plan                               */
  GEMM_E_SIZE = -9,    /* a tile's byte offsets would not fit 31 bits          */
  GEMM_E_WORKSPACE = -10, /* the plan needs a workspace (split K) and none, a
                             smaller or a misaligned one was given            */
  GEMM_E_SCRATCH = -11     /* gemm_run_noalloc: the plan's workspace is larger
                             than GEMM_NOALLOC_SCRATCH_BYTES                  */
};

/* The problem.  M, N >= 0, K >= 0 (K == 0 gives C = epilogue(+0));
 * batch >= 1; with batch > 1, stride_a >= M*K, stride_b >= K*N and
 * stride_c >= M*N.  `tile` selects a tile configuration by id (1 ..
 * gemm_tile_count()), or 0 for the planner's choice; tiles 1-7 and 11-13
 * take 16-bit operands and tiles 8-10 FP8 operands (another gives
 * GEMM_E_ARG).
 * Tile 11 is the persistent short-K kernel (one workgroup per CU looping
 * over 128-row blocks, B held in LDS for the whole launch); it takes only
 * batch 1, 0 < K <= 96 and 0 < N <= 288 with K and N multiples of 8, no
 * bias, GEMM_EPI_NONE or GEMM_EPI_RELU, no split and none of the stage
 * flags (GEMM_E_ARG otherwise), and it gives the same bits as tile 5.  The
 * planner picks it for such problems with at least two blocks per CU.
 * `split_k` cuts K into that many ranges (1 .. 256; fewer if K has fewer
 * trips), or 0 for one range unless GEMM_FLAG_SPLIT_K lets the planner
 * choose. */
typedef struct gemm_desc {
  int64_t M, N, K;
  int32_t in_dtype;  /* GEMM_F16, GEMM_BF16 or GEMM_FP8 (A and B) */
  int32_t out_dtype; /* GEMM_F32, GEMM_F16 or GEMM_BF16 (C)   */
  int32_t epilogue;  /* GEMM_EPI_* activation                   */
  int32_t flags;     /* GEMM_FLAG_* bits                       */
  int64_t batch;
  int64_t stride_a, stride_b, stride_c;
  int32_t tile;
  int32_t split_k;
} gemm_desc;

/* What the planner needs to know about a device (page "Module Tolk.Stage":
 * Renderer.t.async_copy and Renderer.t.shared_max). */
typedef struct gemm_device_caps {
  int32_t num_cus;    /* compute units                                   */
  int32_t lds_bytes;  /* LDS one workgroup may hold (163840 on gfx950)   */
  int32_t async_copy; /* 1: global->LDS copies overlap compute            */
  int32_t wave_size;  /* 64                                               */
  int32_t clock_khz;  /* peak engine clock                                */
  int32_t num_xcds;   /* accelerator complex dies sharing the dispatch    */
  char arch[64];      /* e.g. "gfx950:sramecc+:xnack-"                     */
} gemm_device_caps;

/* A plan's decisions, for tests and reports. */
typedef struct gemm_plan_info {
  int32_t tile_id;
  int32_t bm, bn, bk;       /* workgroup tile                                */
  int32_t waves;            /* waves (64 lanes) per workgroup                */
  int32_t stages;           /* LDS slots in the ring (2..4), 1, or 0 (unstaged) */
  int32_t lds_bytes;        /* LDS the kernel declares                       */
  int32_t vec16;            /* 1: 16-byte copies; 0: element copies          */
  int64_t tiles_m, tiles_n; /* output tiles along M and N (tile 11: 128-row
                               blocks and 1)                                 */
  int64_t workgroups;       /* tiles_m * tiles_n * batch * split_k (tile 11:
                               min(blocks, CUs), each looping over blocks)   */
  int64_t trips;            /* K-trips: ceil(K / bk)                         */
  int64_t mfma_per_run;     /* MFMA instructions one run issues              */
  int32_t mfma_m, mfma_n, mfma_k;
  int32_t split_k;          /* K ranges (1: no split)                        */
  int64_t trips_per_split;  /* trips of each K range (the last may have fewer) */
  int64_t workspace_bytes;  /* device workspace a run needs (0 without split) */
  int64_t tail_rows;        /* > 0: the last tail_rows rows of C run as a second
                               launch with K split into tail_split ranges (the
                               other fields describe the rows above, except
                               workgroups, mfma_per_run and workspace_bytes,
                               which cover both launches); 0: none          */
  int32_t tail_split;       /* K ranges of the tail rows (0 without a tail)  */
  int32_t reserved0;
} gemm_plan_info;

typedef struct gemm_plan_s* gemm_plan_t;

/* Device capabilities of HIP device `device` (host call; no kernel): what the
 * stage rule and the tile choice read about a target (page "Module
 * Tolk.Stage": Renderer.t.async_copy, Renderer.t.shared_max).  Returns
 * GEMM_E_DEVICE, with *out filled as far as known, if the device does not
 * exist or is not a gfx950; GEMM_E_ARG if out is NULL. */
int gemm_device_caps_query(int device, gemm_device_caps* out);

/* Plan for the current HIP device (queries it once per device): the
 * decisions a lowering makes before any launch -- the tile and its wave
 * grid, the number of LDS stages (page "Module Tolk.Stage", depth), the K
 * split, and the grid of ceil(M / BM) x ceil(N / BN) x batch x split_k
 * workgroups (page "gizml:tile", cdiv; the tile program's launch grid).
 * The page's `ir` and `source` likewise fix these per kind and arch with
 * no launch.  Host only: no GPU work, no device memory.  *out receives a new
 * plan the caller owns (gemm_plan_destroy), or NULL on error: GEMM_E_ARG,
 * GEMM_E_DTYPE or GEMM_E_SIZE for a bad description, GEMM_E_DEVICE if the
 * current device is not a gfx950 or no tile fits it, GEMM_E_NOMEM. */
int gemm_plan(const gemm_desc* desc, gemm_plan_t* out);

/* gemm_plan for the given capabilities instead of the current device: no
 * device needed (as the page "gizml:tile", source, lowers for a named
 * kind and arch "with no GPU needed").  Same ownership and errors as
 * gemm_plan; GEMM_E_DEVICE if caps is NULL or not a 64-lane device. */
int gemm_plan_for_caps(const gemm_desc* desc, const gemm_device_caps* caps, gemm_plan_t* out);

/* Copy a plan's decisions out (the fields the page "gizml:tile", ir,
 * reports per node: shape, storage, the mma warp layout).  GEMM_E_PLAN for
 * a NULL plan or a pointer that is not a plan, GEMM_E_ARG if out is NULL. */
int gemm_plan_get_info(gemm_plan_t plan, gemm_plan_info* out);

/* A one-line description (tile, stages, LDS bytes, grid, MFMA shape): the
 * counterpart of the page "gizml:tile", ir (the lowering's decisions as
 * text, the first thing to read when a launch is slower than expected).
 * The string belongs to the plan and lives until gemm_plan_destroy; a NULL
 * plan (or a pointer that is not a plan) gives the static text
 * "(invalid plan)". */
const char* gemm_plan_describe(gemm_plan_t plan);

/* Extra arguments of a run.  bias: device pointer to N fp32 values, needed
 * by plans made with GEMM_FLAG_BIAS (else ignored).  workspace: device
 * memory of at least gemm_plan_info.workspace_bytes bytes, 256-byte aligned,
 * needed by split-K plans (else ignored); its contents on entry do not
 * matter and are overwritten; two runs in flight at once need two
 * workspaces.  Neither may overlap A, B or C. */
typedef struct gemm_run_args {
  const void* bias;
  void* workspace;
  int64_t workspace_bytes;
  int64_t reserved[4]; /* must be 0 */
} gemm_run_args;

/*
 * Launch C = epilogue(A . B) on `stream` (a hipStream_t; NULL = the null
 * stream): the page "gizml:tile", run (the body runs for each point of the
 * grid; the written tensor keeps its values outside what the programs
 * store, Out.put).  A, B, C are device pointers owned by the caller, aligned to
 * their element size; 16-byte-aligned A and B with K and N multiples of 8
 * (16 for FP8: whole 16-byte chunks)
 * take the 16-byte copy path, others take the element path (same bits).
 * Only C's M x N region of each batch item is written.  Returns
 * GEMM_E_ALIAS if C's extent overlaps A's or B's, GEMM_E_DEVICE if the
 * current device is not gfx950 or holds less LDS than the plan needs, and
 * GEMM_E_LAUNCH if the launch fails.  M == 0 or N == 0 launches nothing.
 */
int gemm_run(gemm_plan_t plan, const void* A, const void* B, void* C, void* stream);

/*
 * gemm_run with a bias (page "gizml:tile", Tile.add with a [1, N] row
 * broadcast) and a workspace (args may be NULL for plans that need
 * neither).  A split-K plan launches two kernels on `stream`: the GEMM,
 * which writes each K range's fp32 sums into the workspace, then the
 * reduction, which writes C.  Returns GEMM_E_ARG if the plan needs a bias
 * and none is given (or args->reserved is not 0), GEMM_E_WORKSPACE if it
 * needs a workspace and none, a smaller or a misaligned one is given,
 * GEMM_E_ALIAS if the bias or workspace overlaps A, B or C, and otherwise
 * what gemm_run returns.  gemm_run(plan, ...) is gemm_run_ex(plan, ...,
 * NULL, stream).
 */
int gemm_run_ex(gemm_plan_t plan, const void* A, const void* B, void* C, const gemm_run_args* args,
                void* stream);

/* Bytes of the fixed device array gemm_run_noalloc uses as its workspace
 * (64 MiB: the four K ranges of a 2048 x 2048 fp32 output). */
#define GEMM_NOALLOC_SCRATCH_BYTES (64ll << 20)

/*
 * gemm_run_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same run, with the optional bias (N fp32 values on the
 * device, for plans made with GEMM_FLAG_BIAS, else ignored), where a
 * split-K plan's workspace is a fixed array of GEMM_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends.
 * The call allocates nothing: the array's device address is looked up
 * (hipGetSymbolAddress) on the first call on each device and kept.
 * Returns GEMM_E_SCRATCH, before touching the device, if the plan needs a
 * larger workspace; otherwise what gemm_run_ex returns.  Every call on one
 * GPU shares that GPU's array, which keeps the last call's partial sums:
 * calls that overlap in time on one GPU (two streams, two host threads)
 * race and may return wrong results, so serialise them.  Nothing in the
 * array needs clearing between calls (every partial sum a run reads is
 * written by that run first).
 */
int gemm_run_noalloc(gemm_plan_t plan, const void* A, const void* B, void* C, const void* bias, void* stream);

/*
 * Measure and keep the fastest configuration for a problem (page
 * "gizml:tile", tune: each configuration timed on this GPU for these
 * shapes, the fastest kept, measured once and then cached; every
 * configuration computes the same result, exactly so wherever the sums are
 * exact, and the run may not read what it writes).
 *
 * Candidates are every tile configuration (desc->tile == 0) or the one
 * given; each unsplit and, with GEMM_FLAG_SPLIT_K, split into 2, 4, 8 or 16
 * ranges of at least 4 trips where args->workspace holds the partial sums,
 * or (desc->split_k > 0) split into exactly desc->split_k ranges; with
 * GEMM_FLAG_SPLIT_K, desc->tile == 0 and desc->split_k == 0 also the
 * planner's own plan where it splits K for the bottom rows only
 * (gemm_plan_info.tail_rows > 0) and the workspace holds its partial sums.
 * Each candidate runs once to warm up, then 5 times, each timed with HIP
 * events on `stream`; the smallest time wins.  A and B are read; C and the
 * workspace are written many times; the bias (GEMM_FLAG_BIAS) is read.
 * The call synchronises `stream` and returns a new plan for the winner in
 * *out (the caller destroys it).  The choice of an unrestricted search
 * (desc->tile == 0, desc->split_k == 0) is kept in a process-wide cache
 * keyed by the device's architecture and CU count and by every field of
 * desc but tile, split_k and GEMM_FLAG_TUNED; gemm_plan with
 * GEMM_FLAG_TUNED reads it.  A search restricted to a tile or a split
 * returns its winner without caching it.  Errors: as gemm_plan and gemm_run_ex, and
 * GEMM_E_LAUNCH if timing fails.
 */
int gemm_autotune(const gemm_desc* desc, const void* A, const void* B, void* C, const gemm_run_args* args,
                  void* stream, gemm_plan_t* out);

/* The autotune cache as text, one problem per line (device key, problem
 * fields, chosen tile and split, measured microseconds): write it to
 * `path`, read entries from `path` (added to or replacing those held; a
 * split of 0 stands for the planner's plan with its split tail), or
 * forget every entry.  Return GEMM_OK, or GEMM_E_ARG if the file cannot be
 * opened or a line does not parse. */
int gemm_tune_cache_save(const char* path);
int gemm_tune_cache_load(const char* path);
void gemm_tune_cache_clear(void);
/* Number of entries held. */
int gemm_tune_cache_size(void);

/* Free a plan (NULL is ignored).  A plan is the host-side record of one
 * lowering (page "gizml:tile": a tile program's body runs once and records
 * its IR; here that record is host memory the caller owns).  Runs already
 * queued with it are unaffected (they copied its decisions at launch); the
 * plan may not be used afterwards (a freed plan cannot be detected: no
 * call promises an error for one). */
void gemm_plan_destroy(gemm_plan_t plan);

/* Static text naming an error code: failures are named and specific (page
 * "Module Tolk.Uniform", check: the error names the kernel, the operation
 * and the loop).  Unknown codes give "unknown error code". */
const char* gemm_strerror(int code);

/*
 * The stage-count rule (page "Module Tolk.Stage", depth): with operand tiles
 * of tile_bytes[0 .. n_tiles-1] bytes each and `used` bytes of LDS taken by
 * others, 2 where caps->async_copy and two stages fit caps->lds_bytes, 1
 * where one does, and 0 where neither does, where n_tiles == 0, where a tile
 * holds less than one 16-byte copy, where the device has no LDS or no
 * lanes, or where stage_enabled == 0.
 */
int gemm_stage_depth(const gemm_device_caps* caps, int64_t used, const int64_t* tile_bytes,
                     int n_tiles, int stage_enabled);

/* Number of tile configurations (valid `tile` ids are 1 .. count): the
 * configurations a tuned launch chooses among (page "gizml:tile", tune). */
int gemm_tile_count(void);

/* HIP runtime version the library is running against (hipRuntimeGetVersion),
 * or -1.  A diagnostic of the library with no counterpart on the pages: a
 * process must run the library on the runtime its caller's device pointers
 * and streams come from. */
int gemm_runtime_version(void);

#ifdef __cplusplus
}
#endif

#endif
