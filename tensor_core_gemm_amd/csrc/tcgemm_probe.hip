// Diagnostic kernels that measure gfx950 lane layouts (declared in
// tcgemm_probe.h).  Each launches one workgroup; host wrappers check every
// address against the LDS buffer before launching, so all accesses stay in
// bounds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tcgemm.h"
#include "tcgemm_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;

struct LaneWords {
  uint32_t v[64];
};

__global__ __launch_bounds__(64) void probe_mfma_kernel(int kind, const uint16_t* a, const uint16_t* b,
                                                        float* d) {
  const int l = threadIdx.x;
  u32x4 ar, br;
  for (int i = 0; i < 4; ++i) {
    ar[i] = (uint32_t)a[l * 8 + 2 * i] | ((uint32_t)a[l * 8 + 2 * i + 1] << 16);
    br[i] = (uint32_t)b[l * 8 + 2 * i] | ((uint32_t)b[l * 8 + 2 * i + 1] << 16);
  }
  float out[16];
  for (int i = 0; i < 16; ++i) out[i] = 0.0f;
  if (kind == TCG_PROBE_MFMA_32x32x16_BF16) {
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ar),
                                                  __builtin_bit_cast(bf16x8, br), acc, 0, 0, 0);
    for (int i = 0; i < 16; ++i) out[i] = acc[i];
  } else if (kind == TCG_PROBE_MFMA_32x32x16_F16) {
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, ar),
                                                 __builtin_bit_cast(f16x8, br), acc, 0, 0, 0);
    for (int i = 0; i < 16; ++i) out[i] = acc[i];
  } else if (kind == TCG_PROBE_MFMA_16x16x32_BF16) {
    f32x4 acc = {};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ar),
                                                  __builtin_bit_cast(bf16x8, br), acc, 0, 0, 0);
    for (int i = 0; i < 4; ++i) out[i] = acc[i];
  } else {
    f32x4 acc = {};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ar),
                                                 __builtin_bit_cast(f16x8, br), acc, 0, 0, 0);
    for (int i = 0; i < 4; ++i) out[i] = acc[i];
  }
  for (int i = 0; i < 16; ++i) d[l * 16 + i] = out[i];
}

// One v_mfma_f32_32x32x64_f8f6f4 with both operands in FP8 E4M3 (format
// code 0) and no scaling: per lane 32 operand bytes each, 16 results.
__global__ __launch_bounds__(64) void probe_mfma_f8_kernel(const uint8_t* a, const uint8_t* b, float* d) {
  const int l = threadIdx.x;
  i32x8 ar, br;
  for (int i = 0; i < 8; ++i) {
    uint32_t wa = 0, wb = 0;
    for (int q = 0; q < 4; ++q) {
      wa |= (uint32_t)a[l * 32 + 4 * i + q] << (8 * q);
      wb |= (uint32_t)b[l * 32 + 4 * i + q] << (8 * q);
    }
    ar[i] = (int)wa;
    br[i] = (int)wb;
  }
  f32x16 acc = {};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ar, br, acc, 0, 0, 0, 0, 0, 0);
  for (int i = 0; i < 16; ++i) d[l * 16 + i] = acc[i];
}

constexpr int kTrLdsBytes = 16384;

__global__ __launch_bounds__(64) void probe_tr16_kernel(const uint16_t* init, int n, LaneWords addr,
                                                        uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kTrLdsBytes / 2];
  for (int i = threadIdx.x; i < kTrLdsBytes / 2; i += 64) lds[i] = (i < n) ? init[i] : 0;
  __syncthreads();
  const int l = threadIdx.x;
  const uint32_t byte = addr.v[l];  // checked on the host: 8-aligned and in range
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4_t*)((__attribute__((address_space(3))) char*)lds + byte));
  for (int i = 0; i < 4; ++i) out[l * 4 + i] = (uint16_t)r[i];
}

__global__ __launch_bounds__(64) void probe_tr8_kernel(const uint8_t* init, int n, LaneWords addr,
                                                       uint8_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kTrLdsBytes];
  for (int i = threadIdx.x; i < kTrLdsBytes; i += 64) lds[i] = (i < n) ? init[i] : 0;
  __syncthreads();
  const int l = threadIdx.x;
  const uint32_t byte = addr.v[l];  // checked on the host: 8-aligned and in range
  const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (lds_i32x2_t*)((__attribute__((address_space(3))) char*)lds + byte));
  for (int i = 0; i < 8; ++i) out[l * 8 + i] = (uint8_t)((uint32_t)r[i >> 2] >> (8 * (i & 3)));
}

constexpr int kDmaLdsBytes = 8192;

__global__ __launch_bounds__(64) void probe_buffer_lds_kernel(const uint32_t* src, uint32_t records,
                                                              LaneWords voff, uint32_t base,
                                                              uint32_t* out) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kDmaLdsBytes / 4];
  for (int i = threadIdx.x; i < kDmaLdsBytes / 4; i += 64) lds[i] = 0xDEADBEEFu;
  __syncthreads();
  __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, (int)records, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (lds_void_t*)((__attribute__((address_space(3))) char*)lds + base), 16,
      voff.v[threadIdx.x], 0, 0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = threadIdx.x; i < kDmaLdsBytes / 4; i += 64) out[i] = lds[i];
}

// Clock probe: the first lane of each workgroup records which XCD it runs
// on (the XCC_ID hardware register), the shader-clock counter (s_memtime)
// and the constant-rate counter (s_memrealtime).  Two launches bracketing a
// stretch of work give, per XCD, the average shader clock over it.
__global__ __launch_bounds__(64) void probe_clock_kernel(uint64_t* out) {
  if (threadIdx.x == 0) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    out[3 * blockIdx.x] = xcc & 0xffu;
    out[3 * blockIdx.x + 1] = t;
    out[3 * blockIdx.x + 2] = r;
  }
}

// Sustained MFMA throughput with register operands: no memory traffic, no
// LDS, no barriers inside the loop.  One workgroup of four waves per CU (one
// wave per SIMD, as in the GEMM kernels; the workgroup's LDS reservation
// keeps a second workgroup off the CU), each wave issuing back-to-back MFMAs
// into four independent accumulators while it cycles through eight A and
// eight B operand registers, pairing A register i with B register (i + j)
// mod 8 in round j, so consecutive MFMAs see different values as in a GEMM
// (the shader clock under this load depends on the operand bits).
constexpr int kRateLdsBytes = 96 * 1024;

template <int KIND>
__device__ __forceinline__ void rate_mfma(const u32x4& a, const u32x4& b, f32x16& acc) {
  if constexpr (KIND == TCG_PROBE_MFMA_32x32x16_BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
  } else if constexpr (KIND == TCG_PROBE_MFMA_32x32x16_F16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                 acc, 0, 0, 0);
  } else {
    // the 16x16x32 forms use the first four accumulator registers
    f32x4 c = {acc[0], acc[1], acc[2], acc[3]};
    if constexpr (KIND == TCG_PROBE_MFMA_16x16x32_BF16)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
    else
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
    acc[0] = c[0];
    acc[1] = c[1];
    acc[2] = c[2];
    acc[3] = c[3];
  }
}

// FP8 E4M3 operands: 32 bytes per lane per register set (8 words).
__global__ __launch_bounds__(256) void probe_mfma_rate_f8_kernel(const uint32_t* ops, int iters, float* sink,
                                                                 uint64_t* ticks) {
  __shared__ char reserve[kRateLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  if (iters < 0) ((volatile char*)reserve)[tid] = 0;  // keeps the reservation; never taken
  i32x8 a[8], b[8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      a[r][q] = (int)ops[(r * 64 + lane) * 8 + q];
      b[r][q] = (int)ops[((8 + r) * 64 + lane) * 8 + q];
    }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[(i + j) & 7], acc[i & 3], 0, 0, 0, 0,
                                                                     0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * 256 + tid] = s;
  if (tid == 0) ticks[blockIdx.x] = t1 - t0;
}

template <int KIND>
__global__ __launch_bounds__(256) void probe_mfma_rate_kernel(const uint16_t* ops, int iters, float* sink,
                                                              uint64_t* ticks) {
  __shared__ char reserve[kRateLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  if (iters < 0) ((volatile char*)reserve)[tid] = 0;  // keeps the reservation; never taken
  u32x4 a[8], b[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint16_t* pa = ops + (r * 64 + lane) * 8;
    const uint16_t* pb = ops + ((8 + r) * 64 + lane) * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[r][q] = (uint32_t)pa[2 * q] | ((uint32_t)pa[2 * q + 1] << 16);
      b[r][q] = (uint32_t)pb[2 * q] | ((uint32_t)pb[2 * q + 1] << 16);
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) rate_mfma<KIND>(a[i], b[(i + j) & 7], acc[i & 3]);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * 256 + tid] = s;
  if (tid == 0) ticks[blockIdx.x] = t1 - t0;
}

// Issue cost of global->LDS copies between MFMAs.  One workgroup per CU
// (each reserves 96 KiB of LDS) of NWV waves; every wave runs `iters`
// rounds of 32 back-to-back v_mfma_f32_32x32x16_bf16 on register operands
// (four accumulators), and issues NB bursts of BURST 16-byte-per-lane
// copies into LDS per round, each burst right after an MFMA, bursts evenly
// spaced.  The copies read a 64 KiB buffer (offsets below 64 KiB - 16) and
// write this workgroup's LDS (wave w: 8 KiB at 8 KiB w); a wait for all but
// the last 15 copies closes each round.  The loop is timed with s_memtime
// between two workgroup barriers, so it covers every wave.  Compared with
// the copy-free loop, the time per MFMA shows how long a copy holds up the
// MFMA issue of its wave, and how much a second wave on the SIMD hides.
// With S16 the rounds are 64 v_mfma_f32_16x16x32_bf16 instead (the same
// flops and the same copies per round, so one copy per 8 MFMAs).
constexpr int kCopyProbeLds = 96 * 1024;

template <int NWV, int NB, int BURST, bool S16>
__global__ __launch_bounds__(NWV * 64) void probe_copy_issue_kernel(const uint16_t* ops, const uint32_t* src,
                                                                   int iters, float* sink, uint64_t* ticks) {
  __shared__ __attribute__((aligned(1024))) char lds[kCopyProbeLds];
  constexpr int RM = S16 ? 64 : 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  u32x4 a[4], b[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[r][q] = (uint32_t)ops[(r * 64 + lane) * 8 + 2 * q] | ((uint32_t)ops[(r * 64 + lane) * 8 + 2 * q + 1] << 16);
      b[r][q] = (uint32_t)ops[((4 + r) * 64 + lane) * 8 + 2 * q] |
                ((uint32_t)ops[((4 + r) * 64 + lane) * 8 + 2 * q + 1] << 16);
    }
  f32x16 acc[4];
  f32x4 acc16[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc16[c][r] = 0.0f;
  }
  i32x4 rs;
  {
    const uint64_t base = (uint64_t)src;
    rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    rs[1] = __builtin_amdgcn_readfirstlane((int)((base >> 32) & 0xffffu));
    rs[2] = 65536;
    rs[3] = 0x00020000;
  }
  const uint32_t voff = (uint32_t)(lane * 16 + (w & 3) * 1024);  // + k * 4096 < 65536 - 16
  const uint32_t ldsb = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds + w * 8192;
  constexpr int SP = NB > 0 ? RM / NB : RM;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      if constexpr (S16)
        acc16[m & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[m & 3]),
                                                               __builtin_bit_cast(bf16x8, b[(m >> 2) & 3]),
                                                               acc16[m & 3], 0, 0, 0);
      else
        acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[m & 3]),
                                                             __builtin_bit_cast(bf16x8, b[(m >> 2) & 3]), acc[m & 3],
                                                             0, 0, 0);
      if (NB > 0 && (m % SP) == SP - 1) {
#pragma unroll
        for (int q = 0; q < BURST; ++q) {
          const int k = ((m / SP) * BURST + q) & 7;  // 8 x 1 KiB of LDS per wave
          const uint32_t m0 = __builtin_amdgcn_readfirstlane(ldsb + k * 1024);
          asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                       :
                       : "s"(m0), "v"(voff + k * 4096), "s"(rs)
                       : "memory", "m0");
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (NB > 0) __builtin_amdgcn_s_waitcnt(0xF7F);  // vmcnt(15)
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc16[c][r];
  }
  sink[blockIdx.x * 512 + tid] = s + (float)lds[tid];
  if (tid == 0) ticks[blockIdx.x] = t1 - t0;
}

int launch_status() { return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_E_LAUNCH; }

}  // namespace

extern "C" int tcg_probe_mfma(int kind, const uint16_t* a_regs_dev, const uint16_t* b_regs_dev,
                              float* d_regs_dev, void* stream) {
  if (kind < 0 || kind > 3 || !a_regs_dev || !b_regs_dev || !d_regs_dev) return GEMM_E_ARG;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, kind,
                     a_regs_dev, b_regs_dev, d_regs_dev);
  return launch_status();
}

extern "C" int tcg_probe_ds_read_tr16(const uint16_t* lds_init_dev, int n_elems,
                                      const uint32_t* lane_byte_addr_host, uint16_t* out_dev,
                                      void* stream) {
  if (!lds_init_dev || !lane_byte_addr_host || !out_dev) return GEMM_E_ARG;
  if (n_elems < 0 || n_elems > kTrLdsBytes / 2) return GEMM_E_ARG;
  LaneWords a;
  for (int l = 0; l < 64; ++l) {
    uint32_t v = lane_byte_addr_host[l];
    if ((v & 7u) != 0 || v + 8u > (uint32_t)kTrLdsBytes) return GEMM_E_ARG;
    a.v[l] = v;
  }
  hipLaunchKernelGGL(probe_tr16_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, lds_init_dev,
                     n_elems, a, out_dev);
  return launch_status();
}

extern "C" int tcg_probe_buffer_lds(const uint32_t* src_dev, uint32_t num_records,
                                    const uint32_t* lane_voffset_host, uint32_t lds_byte_base,
                                    uint32_t* out_dev, void* stream) {
  if (!src_dev || !lane_voffset_host || !out_dev) return GEMM_E_ARG;
  if ((lds_byte_base & 15u) != 0 || lds_byte_base + 1024u > (uint32_t)kDmaLdsBytes) return GEMM_E_ARG;
  if (num_records > 0x7fffffffu) return GEMM_E_ARG;
  LaneWords v;
  for (int l = 0; l < 64; ++l) v.v[l] = lane_voffset_host[l];
  hipLaunchKernelGGL(probe_buffer_lds_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, src_dev,
                     num_records, v, lds_byte_base, out_dev);
  return launch_status();
}

extern "C" int tcg_probe_mfma_f8(const uint8_t* a_regs_dev, const uint8_t* b_regs_dev, float* d_regs_dev,
                                 void* stream) {
  if (!a_regs_dev || !b_regs_dev || !d_regs_dev) return GEMM_E_ARG;
  hipLaunchKernelGGL(probe_mfma_f8_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, a_regs_dev, b_regs_dev,
                     d_regs_dev);
  return launch_status();
}

extern "C" int tcg_probe_ds_read_tr8(const uint8_t* lds_init_dev, int n_bytes, const uint32_t* lane_byte_addr_host,
                                     uint8_t* out_dev, void* stream) {
  if (!lds_init_dev || !lane_byte_addr_host || !out_dev) return GEMM_E_ARG;
  if (n_bytes < 0 || n_bytes > kTrLdsBytes) return GEMM_E_ARG;
  LaneWords a;
  for (int l = 0; l < 64; ++l) {
    uint32_t v = lane_byte_addr_host[l];
    if ((v & 7u) != 0 || v + 8u > (uint32_t)kTrLdsBytes) return GEMM_E_ARG;
    a.v[l] = v;
  }
  hipLaunchKernelGGL(probe_tr8_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, lds_init_dev, n_bytes, a,
                     out_dev);
  return launch_status();
}

extern "C" int tcg_probe_clock(int workgroups, uint64_t* out_dev, void* stream) {
  if (workgroups < 1 || workgroups > 65536 || !out_dev) return GEMM_E_ARG;
  hipLaunchKernelGGL(probe_clock_kernel, dim3((uint32_t)workgroups), dim3(64), 0, (hipStream_t)stream, out_dev);
  return launch_status();
}

extern "C" int tcg_probe_wallclock_khz(int device, int* khz) {
  if (!khz) return GEMM_E_ARG;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, device) != hipSuccess) return GEMM_E_DEVICE;
  *khz = v;
  return GEMM_OK;
}

extern "C" int tcg_probe_mfma_rate(int kind, int workgroups, int iters, const uint16_t* operands_dev,
                                   float* sink_dev, uint64_t* ticks_dev, void* stream) {
  if (kind < 0 || kind > TCG_PROBE_MFMA_32x32x64_FP8 || workgroups < 1 || workgroups > 65536 || iters < 0 ||
      !operands_dev ||
      !sink_dev || !ticks_dev)
    return GEMM_E_ARG;
  const dim3 g((uint32_t)workgroups), b(256);
  const hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case TCG_PROBE_MFMA_32x32x16_BF16:
      hipLaunchKernelGGL(probe_mfma_rate_kernel<TCG_PROBE_MFMA_32x32x16_BF16>, g, b, 0, s, operands_dev, iters,
                         sink_dev, ticks_dev);
      break;
    case TCG_PROBE_MFMA_32x32x16_F16:
      hipLaunchKernelGGL(probe_mfma_rate_kernel<TCG_PROBE_MFMA_32x32x16_F16>, g, b, 0, s, operands_dev, iters,
                         sink_dev, ticks_dev);
      break;
    case TCG_PROBE_MFMA_16x16x32_BF16:
      hipLaunchKernelGGL(probe_mfma_rate_kernel<TCG_PROBE_MFMA_16x16x32_BF16>, g, b, 0, s, operands_dev, iters,
                         sink_dev, ticks_dev);
      break;
    case TCG_PROBE_MFMA_16x16x32_F16:
      hipLaunchKernelGGL(probe_mfma_rate_kernel<TCG_PROBE_MFMA_16x16x32_F16>, g, b, 0, s, operands_dev, iters,
                         sink_dev, ticks_dev);
      break;
    default:
      hipLaunchKernelGGL(probe_mfma_rate_f8_kernel, g, b, 0, s, (const uint32_t*)operands_dev, iters, sink_dev,
                         ticks_dev);
      break;
  }
  return launch_status();
}

extern "C" int tcg_probe_copy_issue(int pattern, int workgroups, int iters, const uint16_t* operands_dev,
                                    const uint32_t* src_dev, float* sink_dev, uint64_t* ticks_dev, void* stream) {
  if (workgroups < 1 || workgroups > 65536 || iters < 0 || !operands_dev || !src_dev || !sink_dev || !ticks_dev)
    return GEMM_E_ARG;
  const dim3 g((uint32_t)workgroups);
  const hipStream_t s = (hipStream_t)stream;
#define TCG_COPY_CASE(P, NWV, NB, BURST, S16)                                                             \
  case P:                                                                                                 \
    hipLaunchKernelGGL((probe_copy_issue_kernel<NWV, NB, BURST, S16>), g, dim3(NWV * 64), 0, s, operands_dev, src_dev, \
                       iters, sink_dev, ticks_dev);                                                       \
    break;
  switch (pattern) {
    TCG_COPY_CASE(TCG_PROBE_COPY_4W_NONE, 4, 0, 0, false)
    TCG_COPY_CASE(TCG_PROBE_COPY_4W_8X1, 4, 8, 1, false)
    TCG_COPY_CASE(TCG_PROBE_COPY_4W_2X4, 4, 2, 4, false)
    TCG_COPY_CASE(TCG_PROBE_COPY_8W_NONE, 8, 0, 0, false)
    TCG_COPY_CASE(TCG_PROBE_COPY_8W_4X1, 8, 4, 1, false)
    TCG_COPY_CASE(TCG_PROBE_COPY_8W_8X1, 8, 8, 1, false)
    TCG_COPY_CASE(TCG_PROBE_COPY_4W_NONE_16X16, 4, 0, 0, true)
    TCG_COPY_CASE(TCG_PROBE_COPY_4W_8X1_16X16, 4, 8, 1, true)
    default:
      return GEMM_E_ARG;
  }
#undef TCG_COPY_CASE
  return launch_status();
}
