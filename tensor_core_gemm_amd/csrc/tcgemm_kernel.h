// Device code of the GEMM: C = epilogue(A . B) on gfx950 MFMA units.
//
// One kernel template serves three paths that issue the same MFMA sequence
// on the same values, so their results are bit-identical (page "Module
// Tolk.Stage": staging copies values unchanged):
//
//   STAGES = 2  two LDS slots: chunk t+1 is copied into slot (t+1) mod 2
//               while slot t mod 2 feeds the MFMAs; one barrier per trip
//               (page "Module Tolk.Stage", "Two stages"); tiles built for
//               deeper rings take 3 or 4 slots the same way (page
//               "gizml:tile", Program.stages);
//   STAGES = 1  one slot: copy at the start of the trip, barrier, compute,
//               barrier (the single-stage case of the same page);
//   STAGES = 0  unstaged: every wave loads its fragments straight from
//               global memory, a few bytes at a time (the "Setting.stage
//               off" case); only its output passes through LDS, on the
//               epilogue path all kernels share.
//
// Copies move 16 bytes per lane (VEC16: a buffer load that writes LDS
// directly, gfx950's asynchronous global->LDS copy) or, for operands whose
// rows are not 16-byte aligned, 16 bytes' worth of element loads per lane
// (8 16-bit or 16 FP8 elements) followed by one 16-byte LDS write.  Either way a lane owns the same LDS chunk positions,
// so the LDS image is the same.
//
// Out-of-range elements read 0 (page "gizml:tile", In.at): masked lanes use
// a buffer offset past the resource's size, which the buffer unit turns into
// a zero read.  Out-of-range outputs are not written (Out.put).
//
// Trip counts are the same for every lane of a workgroup, so every barrier
// and MFMA runs in uniform control flow (page "Module Tolk.Uniform").
//
// Split K: with splits > 1 a workgroup folds one range of trips only and
// stores its fp32 sums, unrounded and without the epilogue, into a
// workspace; a reduction kernel adds the ranges in ascending order and
// applies the epilogue.  Every path of one plan splits the same way.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tcgemm_epilogue.h"
#include "tcgemm_kernel_args.h"
#include "tcgemm_layout.h"
#include "tcgemm_tiles.h"

namespace tcg {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x2v lds_i32x2;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr uint32_t kOOB = 0x80000000u;  // a byte offset no resource here reaches

// The LDS layout (swizzles, copy plan, fragment-read addresses) is in
// tcgemm_layout.h, shared with host-side checks.

// ---------------------------------------------------------------------------
// s_waitcnt immediate (gfx9 encoding): vmcnt = N (bits 3:0 and 15:14),
// expcnt unchanged (7), lgkmcnt = 0.
template <int N>
constexpr int waitcnt_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  return (N & 15) | ((N >> 4) << 14) | (7 << 4);
}

// Scheduling of one k-step: the fragment reads of the next k-step (NR LDS
// reads) are issued two at a time between the first MFMAs of this one, so
// they have almost the whole k-step to return; the other MFMAs follow.
template <int NR, int NM>
__device__ __forceinline__ void interleave_reads_into_mfmas() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  constexpr int pairs = (NR + 1) / 2 < NM ? (NR + 1) / 2 : NM;
#pragma unroll
  for (int i = 0; i < pairs; ++i) {
    __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
  }
  if (NM > pairs) __builtin_amdgcn_sched_group_barrier(kMfma, NM - pairs, 0);
}

// A workgroup barrier.  The waits it needs are issued explicitly before it
// (the waitcnt above); the memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void workgroup_barrier() {
  asm volatile("s_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// Buffer resource for raw (unstructured) loads: base address, size in bytes.
// Offsets at or past the size read 0 (the zero-fill of masked lanes).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
  const uint64_t b = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((b >> 32) & 0xffffu));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(n);
  r[3] = 0x00020000;  // raw buffer, 32-bit data format (gfx9)
  return r;
}

// One 16-byte-per-lane copy from a buffer straight into LDS: lane l's 16
// bytes land at lds_base + 16 l.  Issued as inline assembly so that the
// compiler's wait insertion does not track it (it cannot tell the ring's
// slots apart and would drain every copy in flight before some LDS reads);
// the kernel issues the waits these copies need itself (vmcnt before each
// barrier).  The copies are the only vector-memory loads of the staged loop.
__device__ __forceinline__ void copy16_to_lds(const i32x4& rsrc, uint32_t lds_base, uint32_t voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) { return (uint32_t)(uintptr_t)p; }

// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

template <bool BF16IN>
__device__ __forceinline__ f32x16 mfma(const u32x4& src0, const u32x4& src1, const f32x16& acc) {
  if constexpr (BF16IN)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, src0),
                                                   __builtin_bit_cast(bf16x8, src1), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, src0),
                                                  __builtin_bit_cast(f16x8, src1), acc, 0, 0, 0);
}
// FP8 E4M3 operands (format code 0 for both), no scaling: 32 bytes per
// lane, k = 32 (lane / 32) + byte for the row (or column) lane mod 32.
template <bool BF16IN>
__device__ __forceinline__ f32x16 mfma(const u32x8& src0, const u32x8& src1, const f32x16& acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, src0),
                                                         __builtin_bit_cast(i32x8, src1), acc, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return (lo & 0xffffu) | (hi << 16); }
__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  return (b0 & 0xffu) | ((b1 & 0xffu) << 8) | ((b2 & 0xffu) << 16) | (b3 << 24);
}

// One operand element of ES bytes through a buffer resource (zero past its end).
template <int ES>
__device__ __forceinline__ uint32_t load_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (ES == 2)
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  else
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// n elements (16 bytes' worth per 4 words) packed little-endian into words.
template <int ES, int NW>
__device__ __forceinline__ void pack_elems(const uint32_t* e, uint32_t* w) {
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    if constexpr (ES == 2)
      w[q] = pack2(e[2 * q], e[2 * q + 1]);
    else
      w[q] = pack4(e[4 * q], e[4 * q + 1], e[4 * q + 2], e[4 * q + 3]);
  }
}

// ---------------------------------------------------------------------------
// Where a workgroup works: (K range, batch item, tile row, tile column).
struct TilePos {
  int64_t split, b, tm, tn;
};

__device__ __forceinline__ TilePos tile_of(const KArgs& a) {
  // The planner keeps workgroups x lanes below 2^32, so every count here
  // fits 32 bits: 32-bit divisions are a fraction of the scalar code of
  // 64-bit ones, and this runs before the first copy can issue.
  uint32_t wg = blockIdx.x;
  // Workgroups are dealt to the 8 XCDs round-robin; renumber so that the
  // workgroups on one XCD take consecutive tiles (which share A rows and B
  // columns in that XCD's L2).
  if (a.xcd_remap) {
    const uint32_t q = (uint32_t)a.workgroups / 8;
    if (wg < 8 * q) wg = (wg % 8) * q + wg / 8;
  }
  const uint32_t tiles_m = (uint32_t)a.tiles_m, tiles_n = (uint32_t)a.tiles_n;
  const uint32_t per_batch = tiles_m * tiles_n;
  const uint32_t per_split = per_batch * (uint32_t)a.batch;
  TilePos p;
  const uint32_t split = wg / per_split;
  wg -= split * per_split;
  const uint32_t b = wg / per_batch;
  const uint32_t t = wg - b * per_batch;
  // grouped order: group_m tile rows at a time, column-major inside a group
  const uint32_t group_m = (uint32_t)a.group_m;
  const uint32_t in_group = group_m * tiles_n;
  const uint32_t g = t / in_group;
  const uint32_t first = g * group_m;
  const uint32_t gsize = (tiles_m - first) < group_m ? (tiles_m - first) : group_m;
  const uint32_t r = t - g * in_group;
  p.split = split;
  p.b = b;
  p.tm = first + r % gsize;
  p.tn = r / gsize;
  return p;
}


// ---------------------------------------------------------------------------
// Where a workgroup's results go: C of its batch item with the epilogue, or
// (split K) its range's fp32 partial sums with none.
struct OutRef {
  char* C;            // element (0, 0) of the M x N output, row pitch N
  const float* bias;  // or null
  int64_t M, N;
  int dtype;          // kOutF32, kOutF16 or kOutBF16
  int act;
  int vec4, vec16;    // aligned 4-element / 16-byte stores allowed
};

// Whole-vector output stores.  Tiles that run one workgroup per CU write
// their 16-bit outputs with the non-temporal hint: measured 1-2 % faster on
// 4096^3 (bf16 and FP8), where every tile's output leaves at the end of
// the launch; on the tiles that run several workgroups per CU (the Swin
// projection) and on split-K partial sums, which the reduction reads back
// at once, it was slower, so those stores stay plain.
template <bool NT, class V>
__device__ __forceinline__ void store_vec(char* dst, const V& v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, (V*)dst);
  else
    *(V*)dst = v;
}

__device__ __forceinline__ OutRef out_ref(const KArgs& a, const TilePos& tp) {
  OutRef o;
  o.M = a.M;
  o.N = a.N;
  if (a.splits > 1) {
    o.C = (char*)(a.ws + (tp.split * a.batch + tp.b) * a.M * a.N);
    o.bias = nullptr;
    o.dtype = kOutF32;
    o.act = kActNone;
    o.vec4 = o.vec16 = a.ws_vec;
  } else {
    o.C = (char*)a.C + tp.b * a.stride_c * (a.out_dtype == kOutF32 ? 4 : 2);
    o.bias = a.bias;
    o.dtype = a.out_dtype;
    o.act = a.act;
    o.vec4 = a.vec_store4;
    o.vec16 = a.vec_store16;
  }
  return o;
}

// The output path of every kernel: each wave writes a 32-row band of its
// results (EPW columns) into its own LDS region, then reads the band back
// and stores 16 bytes per lane, so each store instruction writes whole row
// segments.  The unstaged kernel shares this path: it stages no operand,
// only its output.
//
// Two forms, chosen per kernel instantiation (GEN_EPI) so that each kernel
// carries one: without a bias, with no activation or relu, the activation
// is applied to the accumulators in place and the band holds rounded
// outputs (the cheap, common case; also the split-K partial sums).
// Otherwise (GEN_EPI) the band holds fp32 sums and the epilogue runs on the
// read-back side, four values per lane at a time: applied in place, its bias
// loads, branches and transcendental functions would be copied into each of
// a wave's 64 groups.

// The rounded epilogue's activation without a branch: fmax(floor, v) with
// floor = +0 is relu (a NaN v gives +0, as Tile.relu requires; -0 gives
// +0), and with floor = a quiet NaN it returns v unchanged (maxNum returns
// the other operand when one is a NaN, and NaN when both are).  A branch
// between two epilogues here made the compiler read every accumulator before
// it and spill.  (This stays a compiler max, not a hand-written v_max: the
// compiler must see the read of an MFMA result to wait for it.)
__device__ __forceinline__ float max_floor(float floor, float v) { return __builtin_fmaxf(floor, v); }
__device__ __forceinline__ float act_floor(int act) {
  return act == kActRelu ? 0.0f : __builtin_bit_cast(float, 0x7fc00000u);
}

// Two fp32 values rounded to nearest-even in one instruction (gfx950's
// packed conversions), the first in the low half.
template <int OUT>
__device__ __forceinline__ uint32_t round2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  if constexpr (OUT == kOutBF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// Rounded band (no bias; activation none or relu), OUT the output type.
// Whole 16-byte chunks of C (o.vec16) leave as buffer stores at 32-bit
// offsets from the band's first element: rows past M lie past the
// resource's end and columns past N get an offset past it, so the buffer
// unit drops both and no lane branches.  Otherwise each chunk is stored
// element by element.
template <class T, int OUT, bool NT>
__device__ __forceinline__ void store_rounded(const OutRef& o, const f32x16 (&acc)[T::FM][T::FN],
                                              int64_t m0, int64_t n0, int lane, int w, lds_char* smem) {
  constexpr int EPW = T::EPW, EPJ = EPW / 32;
  const int64_t M = o.M, N = o.N;
  constexpr int osz = OUT == kOutF32 ? 4 : 2;
  constexpr int pitch = EPW * osz + 16;  // bytes per band row (padded against bank conflicts)
  lds_char* band = smem + w * T::EPI_WAVE_BYTES;
  constexpr int cpr = EPW * osz / 16;  // 16-byte chunks per band row
  constexpr int per_elem = 16 / osz;   // elements per chunk
  const bool buffered = o.vec16 && N * osz * 32 < (int64_t)0x7fffffff;
  constexpr int aux = NT ? 2 : 0;  // the non-temporal cache policy bit
  const float floor = act_floor(o.act);  // uniform: one SGPR
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
#pragma unroll
    for (int jb = 0; jb < T::FN / EPJ; ++jb) {
      // One band at a time: keeps the scheduler from pulling every
      // accumulator out of the AGPRs at once.
      __builtin_amdgcn_sched_barrier(0);
      const int row = lane & 31;
#pragma unroll
      for (int jj = 0; jj < EPJ; ++jj) {
        const int j = jb * EPJ + jj;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = 32 * jj + 8 * g + 4 * (lane >> 5);
          float y[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float v = acc[i][j][4 * g + q];
            y[q] = max_floor(floor, v);  // relu or none
          }
          if constexpr (osz == 4) {
            *(__attribute__((address_space(3))) f32x4*)(band + row * pitch + col * 4) = f32x4{y[0], y[1], y[2], y[3]};
          } else {
            *(__attribute__((address_space(3))) u32x2*)(band + row * pitch + col * 2) =
                u32x2{round2<OUT>(y[0], y[1]), round2<OUT>(y[2], y[3])};
          }
        }
      }
      // Same-wave LDS accesses complete in order: the band is readable now,
      // and the next band's writes come after these reads.
      const int64_t mb = m0 + 32 * i;
      const int64_t nb = n0 + EPW * jb;
      constexpr int chunks = 32 * cpr;
      if (buffered) {
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(o.C + (mb * N + nb) * osz, ((M - mb) * N - nb) * osz);
        const int ncols = (int)(N - nb < EPW ? N - nb : EPW);  // columns of this band inside C
#pragma unroll
        for (int idx = lane; idx < chunks; idx += 64) {
          const int r = idx / cpr;
          const int ch = idx - r * cpr;
          const u32x4 v = *(const lds_u32x4*)(band + r * pitch + ch * 16);
          const int c = ch * per_elem;
          const uint32_t off = c < ncols ? (uint32_t)((r * (int)N + c) * osz) : kOOB;
          __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, aux);
        }
      } else {
#pragma unroll
        for (int idx = lane; idx < chunks; idx += 64) {
          const int r = idx / cpr;
          const int ch = idx - r * cpr;
          const u32x4 v = *(const lds_u32x4*)(band + r * pitch + ch * 16);
          const int64_t m = mb + r;
          const int64_t n = nb + (int64_t)ch * per_elem;
          if (m >= M || n >= N) continue;
          char* dst = o.C + (m * N + n) * osz;
          const int cnt = (int)((N - n) < per_elem ? (N - n) : per_elem);
          if (osz == 4) {
            for (int q = 0; q < cnt; ++q) ((uint32_t*)dst)[q] = v[q];
          } else {
            for (int q = 0; q < cnt; ++q) ((uint16_t*)dst)[q] = (uint16_t)(v[q >> 1] >> (16 * (q & 1)));
          }
        }
      }
    }
  }
}

// fp32 band, epilogue on the read-back side (transcendental activations).
template <class T, bool NT>
__device__ __forceinline__ void store_general(const OutRef& o, const f32x16 (&acc)[T::FM][T::FN],
                                              int64_t m0, int64_t n0, int lane, int w, lds_char* smem) {  constexpr int EPW = T::EPW, EPJ = EPW / 32;
  const int64_t M = o.M, N = o.N;
  constexpr int pitch = EPW * 4 + 16;  // bytes per band row (padded against bank conflicts)
  lds_char* band = smem + w * T::EPI_WAVE_BYTES;
  constexpr int cpr = EPW / 4;  // 16-byte chunks per band row
  const int osz = o.dtype == kOutF32 ? 4 : 2;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
#pragma unroll
    for (int jb = 0; jb < T::FN / EPJ; ++jb) {
      // One band at a time: keeps the scheduler from pulling every
      // accumulator out of the AGPRs at once.
      __builtin_amdgcn_sched_barrier(0);
      const int row = lane & 31;
#pragma unroll
      for (int jj = 0; jj < EPJ; ++jj) {
        const int j = jb * EPJ + jj;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = 32 * jj + 8 * g + 4 * (lane >> 5);
          *(__attribute__((address_space(3))) f32x4*)(band + row * pitch + col * 4) =
              f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
      }
      // Same-wave LDS accesses complete in order: the band is readable now,
      // and the next band's writes come after these reads.
      const int64_t mb = m0 + 32 * i;
      const int64_t nb = n0 + EPW * jb;
      constexpr int chunks = 32 * cpr;
#pragma unroll 2
      for (int idx = lane; idx < chunks; idx += 64) {
        const int r = idx / cpr;
        const int ch = idx - r * cpr;
        const f32x4 v = *(const __attribute__((address_space(3))) f32x4*)(band + r * pitch + ch * 16);
        const int64_t m = mb + r;
        const int64_t n = nb + 4 * ch;
        if (m >= M || n >= N) continue;
        float y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) y[q] = v[q];
        epilogue4(y, o.bias, n, N, o.act);
        char* dst = o.C + (m * N + n) * osz;
        const bool full = o.vec4 && n + 4 <= N;
        if (o.dtype == kOutF32) {
          if (full) {
            store_vec<NT>(dst, f32x4{y[0], y[1], y[2], y[3]});
          } else {
            for (int q = 0; q < 4; ++q)
              if (n + q < N) ((float*)dst)[q] = y[q];
          }
        } else {
          uint16_t h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) h[q] = to_out16(y[q], o.dtype);
          if (full) {
            store_vec<NT>(dst, u32x2{pack2(h[0], h[1]), pack2(h[2], h[3])});
          } else {
            for (int q = 0; q < 4; ++q)
              if (n + q < N) ((uint16_t*)dst)[q] = h[q];
          }
        }
      }
    }
  }
}

template <class T, bool GEN_EPI>
__device__ __forceinline__ void store_through_lds(const OutRef& o, const f32x16 (&acc)[T::FM][T::FN],
                                                  int64_t m0, int64_t n0, int lane, int w, lds_char* smem) {
  constexpr bool NT = T::MIN_WAVES == 1;  // see store_vec
  if constexpr (GEN_EPI) {
    store_general<T, NT>(o, acc, m0, n0, lane, w, smem);  // never split partial sums
  } else {
    // fp32 bands: split partial sums, and fp32 outputs (not measured
    // with the hint; one instantiation serves both)
    if (o.dtype == kOutF32)
      store_rounded<T, kOutF32, false>(o, acc, m0, n0, lane, w, smem);
    else if (o.dtype == kOutBF16)
      store_rounded<T, kOutBF16, NT>(o, acc, m0, n0, lane, w, smem);
    else
      store_rounded<T, kOutF16, NT>(o, acc, m0, n0, lane, w, smem);
  }
}

// ---------------------------------------------------------------------------
// The kernel.
// Tiles small enough in LDS for two workgroups per CU keep their registers
// within half a SIMD's file (min_waves = 2), so that two can run.
template <int TID, int STAGES, bool VEC16, bool BF16IN, bool GEN_EPI>
__global__ __launch_bounds__(Tile<TID>::NT) __attribute__((amdgpu_waves_per_eu(Tile<TID>::MIN_WAVES)))
void gemm_kernel(KArgs a) {
  using T = Tile<TID>;
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK, NW = T::NW, NT = T::NT;
  constexpr int FM = T::FM, FN = T::FN, KS = T::KS, WN = T::WN;
  constexpr int CPR_A = T::CPR_A, CPR_B = T::CPR_B;
  constexpr int ES = T::ES, EPC = T::EPC, MK = T::MK;
  // A fragment / B fragment of one MFMA: 8 16-bit or 32 8-bit values per lane.
  using frag_t = std::conditional_t<ES == 2, u32x4, u32x8>;
  constexpr int FW = ES == 2 ? 4 : 8;  // words per fragment

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (w / WN) * T::WTM;  // wave tile origin inside the workgroup tile
  const int wn0 = (w % WN) * T::WTN;

  const TilePos tp = tile_of(a);
  const int64_t M = a.M, N = a.N, K = a.K;
  const int64_t row0 = tp.tm * BM;
  const int64_t col0 = tp.tn * BN;
  const char* Ab = (const char*)a.A + tp.b * a.stride_a * ES;
  const char* Bb = (const char*)a.B + tp.b * a.stride_b * ES;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;  // Program.zeros

  // This workgroup's K range: trips [kt0, kt0 + trips) of the whole range.
  const int kt0 = (int)tp.split * a.trips_per_split;
  const int trips = (a.trips - kt0) < a.trips_per_split ? (a.trips - kt0) : a.trips_per_split;
  const int64_t kbase = (int64_t)kt0 * BK;
  lds_char* smem_epi = nullptr;
  (void)smem_epi;

  if constexpr (STAGES == 0) {
    // ---------------- unstaged: fragments straight from global memory -----
    __shared__ __attribute__((aligned(1024))) char epi_lds[T::EPI_BYTES];
    smem_epi = (lds_char*)epi_lds;
    for (int t = 0; t < trips; ++t) {
      const int64_t k0 = kbase + (int64_t)t * BK;
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + (row0 * K + k0) * ES, ((M - row0) * K - k0) * ES);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + (k0 * N + col0) * ES, ((K - k0) * N - col0) * ES);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        // this lane's MK/2 consecutive k inside the trip
        const int kk = s * MK + (MK / 2) * (lane >> 5);
        frag_t af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm0 + 32 * i + (lane & 31);
          const bool rok = row0 + r < M;
          const uint32_t off = (uint32_t)(r * K + kk) * ES;
          if constexpr (VEC16) {
            // whole 16-byte chunks (K is a multiple of a chunk)
#pragma unroll
            for (int q = 0; q < FW / 4; ++q) {
              const bool ok = rok && (k0 + kk + q * EPC < K);
              const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? off + 16u * q : kOOB, 0, 0);
#pragma unroll
              for (int w4 = 0; w4 < 4; ++w4) af[i][4 * q + w4] = v[w4];
            }
          } else {
            uint32_t e[MK / 2], wv[FW];
#pragma unroll
            for (int q = 0; q < MK / 2; ++q) {
              const bool ok = rok && (k0 + kk + q < K);
              e[q] = load_elem<ES>(ra, ok ? off + (uint32_t)(ES * q) : kOOB);
            }
            pack_elems<ES, FW>(e, wv);
#pragma unroll
            for (int q = 0; q < FW; ++q) af[i][q] = wv[q];
          }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int c = wn0 + 32 * j + (lane & 31);
          const bool cok = col0 + c < N;
          uint32_t e[MK / 2], wv[FW];
#pragma unroll
          for (int q = 0; q < MK / 2; ++q) {
            const bool ok = cok && (k0 + kk + q < K);
            const uint32_t off = (uint32_t)((kk + q) * N + c) * ES;
            e[q] = load_elem<ES>(rb, ok ? off : kOOB);
          }
          pack_elems<ES, FW>(e, wv);
#pragma unroll
          for (int q = 0; q < FW; ++q) bfr[j][q] = wv[q];
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma<BF16IN>(bfr[j], af[i], acc[i][j]);
      }
    }
  } else {
    // ---------------- staged through LDS ----------------------------------
    // slot0 also holds the epilogue's output bands after the last trip.
    __shared__ __attribute__((aligned(1024))) char slot0[T::SLOT > T::EPI_BYTES ? T::SLOT : T::EPI_BYTES];
    __shared__ __attribute__((aligned(1024))) char slot1[STAGES >= 2 ? T::SLOT : 16];
    __shared__ __attribute__((aligned(1024))) char slot2[STAGES >= 3 ? T::SLOT : 16];
    __shared__ __attribute__((aligned(1024))) char slot3[STAGES >= 4 ? T::SLOT : 16];
    smem_epi = (lds_char*)slot0;

    // Copy plan.  Lane position P = i*NT + tid of a slot's chunk array holds
    // the logical chunk (r, c) of the tile with c = (P mod CPR) ^ swz(r): the
    // swizzle is applied on the global side, so each wave writes 1 KiB of LDS
    // contiguously.  Where NT is a multiple of CPR and of the swizzle period,
    // c does not depend on the round i and the byte offset is a per-lane base
    // plus a uniform step per round.
    //
    // Zero-fill: each trip's buffer resource ends exactly at the operand's
    // last element, so A rows past M and B rows past K are out of range and
    // read 0 by themselves; the K tail of A (last trip) and the N tail of B
    // (last tile column) are masked with an out-of-range offset.
    static_assert(T::CH_A % 64 == 0 && T::CH_B % 64 == 0, "copy rounds are whole waves");
    const bool b_ntail = col0 + BN > N;
    // (swz_a repeats every swz_a_period rows, swz_b every 4 rows)
    constexpr bool SIMPLE_A = (NT % CPR_A == 0) && ((NT / CPR_A) % swz_a_period<CPR_A>() == 0) &&
                              (T::CH_A % NT == 0);
    constexpr bool SIMPLE_B = (NT % CPR_B == 0) && ((NT / CPR_B) % swz_b_period<ES>() == 0) && (T::CH_B % NT == 0);
    // Per-lane chunk of round 0 (rounds add NT / CPR rows).
    const ChunkRC a_ch0 = a_chunk_at<CPR_A>(tid);
    const int a_c80 = EPC * a_ch0.c;
    const uint32_t a_off0 = (uint32_t)(a_ch0.r * K + a_c80) * ES;
    const ChunkRC b_ch0 = b_chunk_at<CPR_B, ES>(tid);
    const int b_c80 = EPC * b_ch0.c;
    const uint32_t b_off0 = (uint32_t)(b_ch0.r * N + b_c80) * ES;
    // Copy chunk (trip) t with element loads (rows not 16-byte aligned).
    auto copy_elements = [&](int t, lds_char* slot) __attribute__((always_inline)) {
      const int64_t k0 = kbase + (int64_t)t * BK;
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab + (row0 * K + k0) * ES, ((M - row0) * K - k0) * ES);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb + (k0 * N + col0) * ES, ((K - k0) * N - col0) * ES);
#pragma unroll
      for (int i = 0; i < T::IA; ++i) {
        if (T::CH_A % NT == 0 || (i * NW + w) * 64 < T::CH_A) {
          const ChunkRC ch = a_chunk_at<CPR_A>(i * NT + tid);
          const int r = ch.r;
          const int ce = EPC * ch.c;
          const uint32_t off = (uint32_t)(r * K + ce) * ES;
          uint32_t e[EPC], wv[4];
#pragma unroll
          for (int q = 0; q < EPC; ++q) {
            const bool ok = k0 + ce + q < K;
            e[q] = load_elem<ES>(ra, ok ? off + (uint32_t)(ES * q) : kOOB);
          }
          pack_elems<ES, 4>(e, wv);
          *(lds_u32x4*)(slot + (i * NW + w) * 1024 + lane * 16) = u32x4{wv[0], wv[1], wv[2], wv[3]};
        }
      }
#pragma unroll
      for (int i = 0; i < T::IB; ++i) {
        if (T::CH_B % NT == 0 || (i * NW + w) * 64 < T::CH_B) {
          const ChunkRC ch = b_chunk_at<CPR_B, ES>(i * NT + tid);
          const int r = ch.r;
          const int ce = EPC * ch.c;
          const uint32_t off = (uint32_t)(r * N + ce) * ES;
          uint32_t e[EPC], wv[4];
#pragma unroll
          for (int q = 0; q < EPC; ++q) {
            const bool ok = col0 + ce + q < N;
            e[q] = load_elem<ES>(rb, ok ? off + (uint32_t)(ES * q) : kOOB);
          }
          pack_elems<ES, 4>(e, wv);
          *(lds_u32x4*)(slot + T::A_BYTES + (i * NW + w) * 1024 + lane * 16) = u32x4{wv[0], wv[1], wv[2], wv[3]};
        }
      }
    };
    // Per-trip copy state and one copy instruction (round q: A rounds
    // first, then B rounds) of the 16-byte path.
    struct CopyCtx {
      int64_t k0;
      bool ktail;
      i32x4 wa, wb;
    };
    auto copy_ctx = [&](int t) __attribute__((always_inline)) {
      CopyCtx c;
      c.k0 = kbase + (int64_t)t * BK;
      c.ktail = c.k0 + BK > K;
      c.wa = make_rsrc_words(Ab + (row0 * K + c.k0) * ES, ((M - row0) * K - c.k0) * ES);
      c.wb = make_rsrc_words(Bb + (c.k0 * N + col0) * ES, ((K - c.k0) * N - col0) * ES);
      return c;
    };
    auto copy_part = [&](const CopyCtx& c, lds_char* slot, int q) __attribute__((always_inline)) {
      if (q < T::IA) {
        const int i = q;
        if (T::CH_A % NT == 0 || (i * NW + w) * 64 < T::CH_A) {  // whole waves only
          int c8;
          uint32_t off;
          if constexpr (SIMPLE_A) {
            c8 = a_c80;
            off = a_off0 + (uint32_t)(i * (NT / CPR_A) * K * ES);
          } else {
            const ChunkRC ch = a_chunk_at<CPR_A>(i * NT + tid);
            c8 = EPC * ch.c;
            off = (uint32_t)(ch.r * K + c8) * ES;
          }
          lds_char* dst = slot + (i * NW + w) * 1024;
          const uint32_t o = (c.ktail && c.k0 + c8 >= K) ? kOOB : off;
          copy16_to_lds(c.wa, __builtin_amdgcn_readfirstlane(lds_addr(dst)), o);
        }
      } else {
        const int i = q - T::IA;
        if (T::CH_B % NT == 0 || (i * NW + w) * 64 < T::CH_B) {
          int c8;
          uint32_t off;
          if constexpr (SIMPLE_B) {
            c8 = b_c80;
            off = b_off0 + (uint32_t)(i * (NT / CPR_B) * N * ES);
          } else {
            const ChunkRC ch = b_chunk_at<CPR_B, ES>(i * NT + tid);
            c8 = EPC * ch.c;
            off = (uint32_t)(ch.r * N + c8) * ES;
          }
          lds_char* dst = slot + T::A_BYTES + (i * NW + w) * 1024;
          const uint32_t o = (b_ntail && col0 + c8 >= N) ? kOOB : off;
          copy16_to_lds(c.wb, __builtin_amdgcn_readfirstlane(lds_addr(dst)), o);
        }
      }
    };
    // Copy chunk (trip) t into a slot.
    auto copy = [&](int t, lds_char* slot) __attribute__((always_inline)) {
      if constexpr (VEC16) {
        const CopyCtx c = copy_ctx(t);
#pragma unroll
        for (int q = 0; q < T::IA + T::IB; ++q) copy_part(c, slot, q);
      } else {
        copy_elements(t, slot);
      }
    };

    // Fragments of one k-step (s) from a slot.  Row pitches in the slot:
    // RA bytes for A, RB bytes for B.
    //
    // 16-bit operands.  A fragment (block i, k-step s): lane l reads row
    // wm0 + 32i + (l mod 32) at logical chunk 2s + l/32, i.e. 8 k-contiguous
    // values.  The row's swizzle depends only on l (wm0 and 32i are
    // multiples of the swizzle period), so the lane's byte offset is
    // a_base[s] + i * 32 * RA.  B fragment (block j, k-step s): column
    // (l mod 32) and 8 k-values 16s + 8(l/32) + e, read as two transposing
    // 4-value reads (h = 0, 1).  ds_read_b64_tr_b16 works on groups of 16
    // lanes: lane x of a group receives element x mod 4 of the reads of lanes
    // 4e + x/4, e = 0..3.  So lane 4e + q reads row e of the group's 4 x 16
    // block at columns 4q .. 4q+3, and lane x receives column x.  The row is
    // 16s + 8(l/32) + 4h + ((l mod 16) / 4), whose swizzle depends only on
    // l, so the lane's byte offset is b_base[j] + (16s + 4h) * RB.
    //
    // FP8 operands (the MFMA pairs byte b of A lane l with byte b of B lane
    // l', l and l' in the same half; k = 32 (l / 32) + b is the order used).
    // A fragment: row wm0 + 32i + (l mod 32), bytes 64s + 32(l/32) .. +31:
    // logical chunks 4s + 2(l/32) and the next (two 16-byte reads; the XOR
    // keeps the pair, so the second is the first with bit 4 flipped).  B
    // fragment: column c = l mod 32, 32 k-values in four transposing 8-byte
    // reads t = 0..3.  ds_read_b64_tr_b8 works on groups of 16 lanes: lane x
    // receives byte x mod 8 of the reads of lanes 2e + x/8, e = 0..7.  So
    // lane s of a group reads row 8t + s/2 (+ 32(l/32) + 64s_k) at the 8
    // columns starting 16((l/16) mod 2) + 8(s mod 2) of the block, and lane
    // x receives column x, rows 8t .. 8t+7 in order.  The swizzle of the row
    // depends only on l (rows step by 8), so the lane's byte offset is
    // b_base[j] + (64 s_k + 8t) * RB.
    constexpr int RA = BK * ES, RB = BN * ES;
    static_assert(32 % swz_a_period<CPR_A>() == 0, "A fragment rows must start on a swizzle period");
    static_assert(RA == CPR_A * 16 && RB == CPR_B * 16, "row pitches are whole chunks");
    int a_base[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) a_base[s] = a_frag_base<CPR_A, ES>(lane, s, wm0);
    int b_base[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) b_base[j] = b_frag_base<CPR_B, ES>(lane, j, wn0);
    struct Frags {
      frag_t a[FM], b[FN];
    };
    // Single fragment reads (read r of a k-step: the A reads first, then
    // the B reads) and single MFMAs, for hand-interleaving.
    constexpr int RPA = ES == 2 ? 1 : 2;  // reads per A fragment
    constexpr int RPB = ES == 2 ? 2 : 4;  // reads per B fragment
    constexpr int NREADS = RPA * FM + RPB * FN;
    auto load_one = [&](const lds_char* slot, int s, Frags& f, int r) __attribute__((always_inline)) {
      if (r < RPA * FM) {
        const int i = r / RPA, q = r % RPA;
        const u32x4 v = *(const lds_u32x4*)(slot + ((a_base[s] + i * (32 * RA)) ^ (16 * q)));
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) f.a[i][4 * q + w4] = v[w4];
      } else {
        const int j = (r - RPA * FM) / RPB, h = (r - RPA * FM) % RPB;
        if constexpr (ES == 2) {
          const lds_char* p = slot + T::A_BYTES + b_base[j] + b_frag_row<ES>(s, h) * RB;
          const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
          f.b[j][2 * h] = pack2((uint16_t)x[0], (uint16_t)x[1]);
          f.b[j][2 * h + 1] = pack2((uint16_t)x[2], (uint16_t)x[3]);
        } else {
          const lds_char* p = slot + T::A_BYTES + b_base[j] + b_frag_row<ES>(s, h) * RB;
          const i32x2v x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
          f.b[j][2 * h] = (uint32_t)x[0];
          f.b[j][2 * h + 1] = (uint32_t)x[1];
        }
      }
    };
    auto load = [&](const lds_char* slot, int s, Frags& f) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < NREADS; ++r) load_one(slot, s, f, r);
    };
    // MFMA order within a k-step: B block outer, A block inner, so
    // consecutive MFMAs share their first operand (measured about 2 % faster
    // than the transposed order on bf16 4096^3).  Each accumulator still
    // takes its k-steps in ascending order.
    // The A blocks run up for even B blocks and down for odd ones, so that
    // the two MFMAs on either side of a B change share their A operand too.
    auto mma_one = [&](const Frags& f, int m) __attribute__((always_inline)) {
      const int j = m / FM, i = (j & 1) ? FM - 1 - m % FM : m % FM;
      acc[i][j] = mfma<BF16IN>(f.b[j], f.a[i], acc[i][j]);
    };
    auto mma = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < FM * FN; ++m) mma_one(f, m);
    };
    auto wait_all_and_barrier = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());
      workgroup_barrier();
    };

    Frags f0, f1;
    if constexpr (STAGES >= 2) {
      // A ring of S slots.  Trip t reads slot t mod S while chunks t+1 ..
      // t+S-1 are in flight into the other slots.  With S = 2 this is the
      // two-stage pipeline of the page "Module Tolk.Stage"; more stages hide
      // longer memory latency at the cost of LDS (page "gizml:tile",
      // Program.stages).
      //
      // The one barrier of a trip comes after the last k-step's fragments
      // are in registers and this wave's copy of chunk t+1 has landed: it
      // retires every read of slot t mod S and publishes chunk t+1.  Right
      // after it the slot just retired is refilled with chunk t+S, so every
      // copy has S-1 whole trips to land; then the first fragments of chunk
      // t+1 load while the last k-step's MFMAs run.  Vector-memory loads
      // complete in order, so "chunk t+1 has landed" is a wait until at most
      // the copies of the newer chunks (NDMA instructions each) are
      // outstanding.  Where a copy round is partial (CH not a multiple of
      // NT) the first waves issue one instruction more per chunk than the
      // last; NDMA counts only the instructions every wave issues, so a wave
      // with more waits a little longer than it must, and none too little.
      constexpr int S = STAGES;
      static_assert(S == 2 || (T::CH_A % NT == 0 && T::CH_B % NT == 0),
                    "rings deeper than two need whole copy rounds per wave");
      constexpr int NDMA = T::CH_A / NT + T::CH_B / NT;  // copies every wave issues per chunk
      lds_char* const ring[4] = {(lds_char*)slot0, (lds_char*)slot1, (lds_char*)slot2, (lds_char*)slot3};
      auto wait_newer_and_barrier = [&](int newer) __attribute__((always_inline)) {
        // newer: copies of chunks after the awaited one still allowed in flight
        if (S >= 4 && newer >= 3) {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<(S >= 4 ? 3 : 0) * NDMA>());
        } else if (S >= 3 && newer >= 2) {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<(S >= 3 ? 2 : 0) * NDMA>());
        } else if (newer >= 1) {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<NDMA>());
        } else {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());
        }
        workgroup_barrier();
      };
      auto newest_issued = [&](int t) { return (t + S - 1 < trips ? t + S - 1 : trips - 1); };
      // The 16-byte copies of one chunk go out in NPART parts, so that the
      // address unit never receives a whole chunk's instructions inside one
      // k-step: part 0 right after the barrier that frees the slot
      // (interleaved with the last k-step's MFMAs), part p >= 1 with k-step
      // p - 1 of the next trip.  "pend" marks a trip whose previous trip left
      // parts 1 .. NPART-1 to issue (chunk t - 1 + S, slot t - 1 mod S).  The
      // last part must still land before the barrier that publishes its
      // chunk, S - 2 whole trips plus KS - NPART + 1 k-steps after it
      // issues.  With two k-steps per trip and two slots a second part
      // would have a single k-step, too short (measured slower on the
      // 32-deep 16-bit and the FP8 tiles): there the whole chunk goes out
      // after the barrier.
      constexpr bool SPREAD = VEC16 && (KS >= 3 || S >= 3);
      constexpr int NPART = SPREAD ? 2 : 1;
      static_assert(NPART <= KS, "every part after the first needs a k-step of the next trip");
      constexpr int ND = T::IA + T::IB, NM = FM * FN;
      constexpr int RPM = (NREADS + NM - 1) / NM;
      // copy instructions [part_lo(p), part_lo(p + 1)) form part p
      auto part_lo = [](int p) constexpr { return p * ND / NPART; };
      // Part p of chunk u into slot, one instruction before MFMA m of a
      // k-step when m is the instruction's share of the k-step.
      auto copy_part_at = [&](const CopyCtx& c, lds_char* slot, int p, int m) __attribute__((always_inline)) {
        // the part's instructions q with q * NM / n == m (rounded down),
        // computed rather than searched so the unroller sees a small body
        const int q0 = part_lo(p), n = part_lo(p + 1) - q0;
        const int lo = (m * n + NM - 1) / NM, hi = ((m + 1) * n + NM - 1) / NM;
#pragma unroll
        for (int q = lo; q < hi; ++q) copy_part(c, slot, q0 + q);
      };
      auto rest_of_previous = [&](int t, int j) __attribute__((always_inline)) {
        const CopyCtx c = copy_ctx(t - 1 + S);
#pragma unroll
        for (int q = part_lo(1); q < ND; ++q) copy_part(c, ring[(j + S - 1) % S], q);
      };
      auto trip = [&](int t, auto J, bool pend) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        lds_char* cur = ring[j];
        lds_char* nxt = ring[(j + 1) % S];
        if constexpr (SPREAD) {
          if (pend) rest_of_previous(t, j);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          Frags& now = (s & 1) ? f1 : f0;
          Frags& next = (s & 1) ? f0 : f1;
          if (s + 1 < KS) {
            load(cur, s + 1, next);
            mma(now);
            interleave_reads_into_mfmas<NREADS, FM * FN>();
          } else {
            const int newer = newest_issued(t) - (t + 1);
            wait_newer_and_barrier(newer > 0 ? newer : 0);
            if (t + S < trips) copy(t + S, cur);
            if (t + 1 < trips) load(nxt, 0, next);
            mma(now);
            interleave_reads_into_mfmas<NREADS, FM * FN>();
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // The same trip where chunk t+S exists and chunk t+1 follows (every
      // trip but the last S): the first and the last k-step are interleaved
      // by hand, fragment reads and copy instructions spread between
      // consecutive MFMAs, so the MFMA pipe keeps running while they issue.
      auto trip_fast = [&](int t, auto J, auto PEND) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        constexpr bool pend = decltype(PEND)::value;
        lds_char* cur = ring[j];
        lds_char* nxt = ring[(j + 1) % S];
#pragma unroll
        for (int s = 0; s + 1 < KS; ++s) {
          Frags& now = (s & 1) ? f1 : f0;
          Frags& next = (s & 1) ? f0 : f1;
          if (pend && s + 1 < NPART) {
            const CopyCtx c = copy_ctx(t - 1 + S);
            lds_char* prev = ring[(j + S - 1) % S];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
#pragma unroll
              for (int r = m * RPM; r < (m + 1) * RPM && r < NREADS; ++r) load_one(cur, s + 1, next, r);
              copy_part_at(c, prev, s + 1, m);
              mma_one(now, m);
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
            load(cur, s + 1, next);
            mma(now);
            interleave_reads_into_mfmas<NREADS, FM * FN>();
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        Frags& now = ((KS - 1) & 1) ? f1 : f0;
        Frags& next = ((KS - 1) & 1) ? f0 : f1;
        const int newer = newest_issued(t) - (t + 1);
        wait_newer_and_barrier(newer > 0 ? newer : 0);
        const CopyCtx c = copy_ctx(t + S);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
          for (int r = m * RPM; r < (m + 1) * RPM && r < NREADS; ++r) load_one(nxt, 0, next, r);
          copy_part_at(c, cur, 0, m);
          mma_one(now, m);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (trips > 0) {
#pragma unroll
        for (int c = 0; c < S; ++c)
          if (c < trips) copy(c, ring[c]);
        const int newer = (S - 1 < trips - 1 ? S - 1 : trips - 1);
        wait_newer_and_barrier(newer);
        load(ring[0], 0, f0);
      }
      // Unrolled by S so that each copy and each read names one slot; the
      // last trips are peeled so the loop body has no branch around a whole
      // trip.  KS is even, so every trip starts with its fragments in f0.
      static_assert(KS % 2 == 0, "k-steps per trip must be even");
      static_assert(KS >= 2, "the first k-step of a fast trip is not its last");
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      using Yes = std::true_type;
      using No = std::false_type;
      int t = 0;
      bool pend = false;
      if constexpr (SPREAD) {
        // the first fast trip has no parts of an earlier chunk to issue
        if (2 * S <= trips) {
          trip_fast(0, I0{}, No{});
          trip_fast(1, I1{}, Yes{});
          if constexpr (S >= 3) trip_fast(2, I2{}, Yes{});
          if constexpr (S >= 4) trip_fast(3, I3{}, Yes{});
          for (t = S; t + 2 * S <= trips; t += S) {
            trip_fast(t, I0{}, Yes{});
            trip_fast(t + 1, I1{}, Yes{});
            if constexpr (S >= 3) trip_fast(t + 2, I2{}, Yes{});
            if constexpr (S >= 4) trip_fast(t + 3, I3{}, Yes{});
          }
          pend = true;
        }
      } else if constexpr (VEC16) {
        for (; t + 2 * S <= trips; t += S) {
          trip_fast(t, I0{}, No{});
          trip_fast(t + 1, I1{}, No{});
          if constexpr (S >= 3) trip_fast(t + 2, I2{}, No{});
          if constexpr (S >= 4) trip_fast(t + 3, I3{}, No{});
        }
      }
      for (; t + S <= trips; t += S) {
        trip(t, I0{}, pend);
        trip(t + 1, I1{}, false);
        if constexpr (S >= 3) trip(t + 2, I2{}, false);
        if constexpr (S >= 4) trip(t + 3, I3{}, false);
        pend = false;
      }
      if (t < trips) trip(t, I0{}, pend);
      if constexpr (S >= 3) {
        if (t + 1 < trips) trip(t + 1, I1{}, false);
      }
      if constexpr (S >= 4) {
        if (t + 2 < trips) trip(t + 2, I2{}, false);
      }
    } else {
      for (int t = 0; t < trips; ++t) {
        copy(t, (lds_char*)slot0);
        wait_all_and_barrier();  // publishes the tile
        load((lds_char*)slot0, 0, f0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          Frags& now = (s & 1) ? f1 : f0;
          Frags& next = (s & 1) ? f0 : f1;
          if (s + 1 < KS) load((lds_char*)slot0, s + 1, next);
          mma(now);
        }
        wait_all_and_barrier();  // retires the reads before the next copy
      }
    }
  }

  // ------- epilogue: bias, activation, rounding, masked store (or the -------
  // ------- unrounded partial sums of this K range)                    -------
  // Lane l of MFMA block (i, j) holds, in registers 4g .. 4g+3, the four
  // consecutive columns 8g + 4(l/32) + 0..3 of row (l mod 32).
  const OutRef o = out_ref(a, tp);
  store_through_lds<T, GEN_EPI>(o, acc, row0 + wm0, col0 + wn0, lane, w, smem_epi);
}

// Launch one instantiation: returns hipGetLastError's result.
template <int TID, int STAGES, bool VEC16, bool BF16IN, bool GEN_EPI>
hipError_t launch_one(const KArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_kernel<TID, STAGES, VEC16, BF16IN, GEN_EPI>), dim3((uint32_t)a.workgroups),
                     dim3(Tile<TID>::NT), 0, stream, a);
  return hipGetLastError();
}

// FP8 tiles have one MFMA for their one input type; BF16IN is false there.
template <int TID, bool GEN_EPI>
hipError_t launch_tile(int stages, bool vec16, bool bf16, const KArgs& a, hipStream_t s) {
  constexpr bool kFp8 = Tile<TID>::ES == 1;
#define TCG_CASE(ST)                                                                  \
  if (stages == ST) {                                                                 \
    if constexpr (kFp8) {                                                             \
      return vec16 ? launch_one<TID, ST, true, false, GEN_EPI>(a, s)                  \
                   : launch_one<TID, ST, false, false, GEN_EPI>(a, s);                \
    } else {                                                                          \
      if (vec16) return bf16 ? launch_one<TID, ST, true, true, GEN_EPI>(a, s)         \
                             : launch_one<TID, ST, true, false, GEN_EPI>(a, s);       \
      return bf16 ? launch_one<TID, ST, false, true, GEN_EPI>(a, s)                   \
                  : launch_one<TID, ST, false, false, GEN_EPI>(a, s);                 \
    }                                                                                 \
  }
  TCG_CASE(0)
  TCG_CASE(1)
  TCG_CASE(2)
  if constexpr (Tile<TID>::MAX_STAGES >= 3) { TCG_CASE(3) }
  if constexpr (Tile<TID>::MAX_STAGES >= 4) { TCG_CASE(4) }
#undef TCG_CASE
  return hipErrorInvalidValue;
}

}  // namespace tcg
