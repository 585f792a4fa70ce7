/*
 * tcgemm_probe.h -- diagnostic kernels that pin the gfx950 lane layouts the
 * GEMM kernels rely on.  They are part of libtcgemm.so but not of the GEMM
 * path; the tests call them to check, on the hardware, the assumptions the
 * fragment loaders make.
 *
 * All pointers named *_dev are device memory owned by the caller; *_host
 * arguments are host memory read before the call returns.  Every function
 * launches one workgroup on `stream` (a hipStream_t, or NULL for the null
 * stream), returns 0 on success or a negative GEMM_E_* code (tcgemm.h), and
 * does not synchronise.  Host-side checks reject any address that would fall
 * outside the probe's LDS buffer, so every probe stays in bounds.
 *
 * Why these exist: the page "Module Tolk.Stage" has the cores read their
 * fragments back from the staged (swizzled) tile, and the TVM page on
 * ldmatrix/stmatrix lowering describes fragment loads as warp-collective
 * 8x8 tile moves with a transposing form for the column-major side.  On
 * gfx950 the matching tools are the MFMA operand layouts, the transposing
 * LDS read ds_read_b64_tr_b16 and the buffer load that writes LDS directly;
 * their lane mappings are measured here instead of assumed.
 */
#ifndef TCGEMM_PROBE_H
#define TCGEMM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA shapes a probe can run. */
enum {
  TCG_PROBE_MFMA_32x32x16_BF16 = 0,
  TCG_PROBE_MFMA_32x32x16_F16 = 1,
  TCG_PROBE_MFMA_16x16x32_BF16 = 2,
  TCG_PROBE_MFMA_16x16x32_F16 = 3,
  TCG_PROBE_MFMA_32x32x64_FP8 = 4 /* tcg_probe_mfma_rate only: f8f6f4, both operands E4M3, unscaled */
};

/*
 * One wave runs one MFMA with a zero accumulator.  a_regs_dev and b_regs_dev
 * hold, per lane (64), the 8 16-bit operand values of that lane's source
 * registers (lane-major: [64][8]); d_regs_dev receives per lane the 16 fp32
 * result registers ([64][16]; the 16x16 shapes fill the first 4).
 */
int tcg_probe_mfma(int kind, const uint16_t* a_regs_dev, const uint16_t* b_regs_dev,
                   float* d_regs_dev, void* stream);

/*
 * ds_read_b64_tr_b16: the LDS buffer (16 KiB) is filled from lds_init_dev
 * (n_elems 16-bit values, n_elems <= 8192), then each lane of one wave
 * issues the transposing read at its byte address lane_byte_addr_host[lane]
 * (8-byte aligned, + 8 <= 16384).  out_dev receives the 4 16-bit values each
 * lane gets back ([64][4]).
 */
int tcg_probe_ds_read_tr16(const uint16_t* lds_init_dev, int n_elems,
                           const uint32_t* lane_byte_addr_host, uint16_t* out_dev, void* stream);

/*
 * Buffer load of 16 bytes per lane written straight to LDS.  The LDS buffer
 * (8 KiB) is first filled with 0xDEADBEEF; then one wave loads from a buffer
 * resource whose base is src_dev and whose size is num_records bytes, lane
 * `l` at byte offset lane_voffset_host[l] (offsets >= num_records are out of
 * range and must read 0; the caller keeps every offset + 16 within the
 * memory src_dev really owns), with the LDS destination base lds_byte_base
 * (16-byte aligned, + 1024 <= 8192).  The whole 8 KiB of LDS is then copied
 * to out_dev (2048 words).
 */
int tcg_probe_buffer_lds(const uint32_t* src_dev, uint32_t num_records,
                         const uint32_t* lane_voffset_host, uint32_t lds_byte_base,
                         uint32_t* out_dev, void* stream);

/*
 * One wave runs one v_mfma_f32_32x32x64_f8f6f4 with both operands in FP8
 * E4M3 (format code 0), no scaling and a zero accumulator.  a_regs_dev and
 * b_regs_dev hold, per lane (64), the 32 operand bytes of that lane's 8
 * source registers (lane-major: [64][32], byte 4i+q is byte q of register
 * i); d_regs_dev receives per lane the 16 fp32 result registers ([64][16]).
 */
int tcg_probe_mfma_f8(const uint8_t* a_regs_dev, const uint8_t* b_regs_dev, float* d_regs_dev, void* stream);

/*
 * ds_read_b64_tr_b8: the LDS buffer (16 KiB) is filled from lds_init_dev
 * (n_bytes bytes, n_bytes <= 16384), then each lane of one wave issues the
 * transposing read at its byte address lane_byte_addr_host[lane] (8-byte
 * aligned, + 8 <= 16384).  out_dev receives the 8 bytes each lane gets back
 * ([64][8], byte 4i+q is byte q of result register i).
 */
int tcg_probe_ds_read_tr8(const uint8_t* lds_init_dev, int n_bytes, const uint32_t* lane_byte_addr_host,
                          uint8_t* out_dev, void* stream);

/*
 * Measurement probes (not layout probes): they launch many workgroups.
 *
 * tcg_probe_clock: `workgroups` workgroups of one wave; the first lane of
 * workgroup g writes out_dev[3g] = the XCD it ran on (the XCC_ID hardware
 * register), out_dev[3g+1] = the shader-clock counter (s_memtime) and
 * out_dev[3g+2] = the constant-rate counter (s_memrealtime), whose rate
 * tcg_probe_wallclock_khz reports.  out_dev holds 3 * workgroups values
 * (device memory, caller-owned).  Two launches around a stretch of work on
 * one stream give, per XCD, the average shader clock over that stretch
 * (difference of s_memtime over difference of s_memrealtime, times the
 * constant rate).  1 <= workgroups <= 65536, else GEMM_E_ARG.
 */
int tcg_probe_clock(int workgroups, uint64_t* out_dev, void* stream);

/* The constant rate of s_memrealtime on `device`, in kHz (hipDeviceAttributeWallClockRate).
 * Host only; GEMM_E_DEVICE if the runtime cannot report it. */
int tcg_probe_wallclock_khz(int device, int* khz);

/*
 * Sustained MFMA throughput with operands in registers (no memory traffic
 * inside the loop): `workgroups` workgroups of four waves, one wave per SIMD
 * (each workgroup reserves 96 KiB of LDS, so at most one runs per CU).  Each
 * wave loads 16 operand register sets of 8 16-bit values per lane from
 * operands_dev ([16][64][8] values; for TCG_PROBE_MFMA_32x32x64_FP8, 32
 * bytes per lane and set, [16][64][32] bytes: sets 0-7 are A, 8-15 are B; the
 * caller draws them, e.g. Gaussian, since the clock under MFMA load depends
 * on the operand bits), then runs `iters` rounds of 64 MFMAs of shape `kind`
 * (TCG_PROBE_MFMA_*) into four independent accumulators, pairing A register
 * i with B register (i + j) mod 8 in round j.  sink_dev receives one float
 * per lane (workgroups * 256), so no MFMA is dead code; ticks_dev receives,
 * per workgroup, the shader-clock cycles (s_memtime) of wave 0's loop.
 * Flops per launch: workgroups * 4 * iters * 64 * (32768 for 32x32x16,
 * 16384 for 16x16x32, 131072 for the FP8 32x32x64).  GEMM_E_ARG on a bad
 * kind, count or null pointer.
 */
int tcg_probe_mfma_rate(int kind, int workgroups, int iters, const uint16_t* operands_dev, float* sink_dev,
                        uint64_t* ticks_dev, void* stream);

/* Copy-issue patterns of tcg_probe_copy_issue: waves per workgroup (one per
 * SIMD with 4, two with 8) and 16-byte-per-lane global->LDS copies per
 * round of 32 MFMAs per wave (NxB: N bursts of B copies). */
enum {
  TCG_PROBE_COPY_4W_NONE = 0, /* 4 waves, no copies (the MFMA-only reference) */
  TCG_PROBE_COPY_4W_8X1 = 1,  /* 4 waves, 8 copies, one every 4 MFMAs (the 256x256 tile's rate) */
  TCG_PROBE_COPY_4W_2X4 = 2,  /* 4 waves, 8 copies in 2 bursts of 4 */
  TCG_PROBE_COPY_8W_NONE = 3, /* 8 waves, no copies */
  TCG_PROBE_COPY_8W_4X1 = 4,  /* 8 waves, 4 copies each: the same copies per SIMD as pattern 1 */
  TCG_PROBE_COPY_8W_8X1 = 5,  /* 8 waves, 8 copies each: twice pattern 1's copies per SIMD */
  /* the same two loops as patterns 0 and 1 with 64 v_mfma_f32_16x16x32_bf16
   * per round (the same flops and copies per round; one copy per 8 MFMAs) */
  TCG_PROBE_COPY_4W_NONE_16X16 = 6,
  TCG_PROBE_COPY_4W_8X1_16X16 = 7
};

/*
 * How long a global->LDS copy holds up MFMA issue: `workgroups` workgroups
 * (one per CU: each reserves 96 KiB of LDS) of 4 or 8 waves run `iters`
 * rounds of 32 back-to-back v_mfma_f32_32x32x16_bf16 (or 64
 * v_mfma_f32_16x16x32_bf16) per wave on register operands, with the copies
 * of `pattern` (TCG_PROBE_COPY_*) in between.
 * operands_dev: [8][64][8] 16-bit values (A registers 0-3, B 4-7); src_dev:
 * 64 KiB of device memory the copies read (caller-owned); sink_dev: 512
 * floats per workgroup; ticks_dev: per workgroup, the shader-clock cycles
 * (s_memtime) of the loop, taken between two workgroup barriers so they
 * cover every wave.  Cycles per MFMA per SIMD = ticks / (iters * R * waves
 * per SIMD), R = 32 MFMAs per round (64 for the 16X16 patterns).
 * GEMM_E_ARG on a bad pattern, count or null pointer.
 */
int tcg_probe_copy_issue(int pattern, int workgroups, int iters, const uint16_t* operands_dev,
                         const uint32_t* src_dev, float* sink_dev, uint64_t* ticks_dev, void* stream);

#ifdef __cplusplus
}
#endif

#endif
