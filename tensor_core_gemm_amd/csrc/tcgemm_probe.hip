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
