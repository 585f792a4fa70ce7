// Tile configurations shared by the planner (host) and the kernels (device).
//
// A workgroup computes a BM x BN block of C with WM x WN waves (64 lanes
// each); each wave owns a (BM/WM) x (BN/WN) sub-block made of 32 x 32 MFMA
// blocks.  Tiles 1-7 take 16-bit operands (fp16, bf16), tiles 8-10 take
// 8-bit FP8 E4M3 operands (esize 1): BK counts elements, so an FP8 slot of
// BK = 128 holds as many bytes as a 16-bit one of BK = 64.  K advances BK per trip (page "gizml:tile": the worked example
// folds over K in blocks; page "Module Tolk.Stage", tile: a workgroup of
// 2 x 2 warps, K unrolled per trip).  On gfx950 a compute unit also has four
// SIMDs, so 2 x 2 waves per workgroup keeps one wave on each.
#pragma once

#include <stdint.h>

namespace tcg {

struct TileDesc {
  int id;
  int bm, bn, bk;
  int wm, wn;      // wave grid
  int max_stages;  // deepest LDS ring the kernel is built for
  int min_waves;   // waves per SIMD the register budget must allow (workgroups per CU)
  int esize;       // operand element bytes: 2 (fp16, bf16) or 1 (FP8 E4M3)
  int persistent;  // 1: the persistent short-K kernel (bk, bn: the largest K and N it takes)
};

// id 0 is "planner's choice" in the ABI; real ids start at 1.
constexpr TileDesc kTiles[] = {
    {1, 256, 256, 64, 2, 2, 2, 1, 2},   // wave 128 x 128: large MFMA-bound products
    {2, 128, 128, 64, 2, 2, 2, 2, 2},   // wave 64 x 64: mid sizes / more workgroups
    {3, 64, 64, 64, 2, 2, 3, 2, 2},     // wave 32 x 32: small and ragged products, up to 3 slots
    {4, 256, 96, 32, 4, 1, 2, 2, 2},    // wave 64 x 96: short-K, N a multiple of 96
    {5, 128, 288, 32, 4, 1, 2, 1, 2},   // wave 32 x 288: short-K, N = 288 in one tile
    {6, 256, 256, 32, 2, 2, 4, 1, 2},   // wave 128 x 128, half-depth slots: up to 4 in flight
    {7, 128, 128, 32, 2, 2, 4, 2, 2},   // wave 64 x 64, half-depth slots: up to 4 in flight
    {8, 256, 256, 128, 2, 2, 2, 1, 1},  // FP8, wave 128 x 128
    {9, 128, 128, 128, 2, 2, 2, 2, 1},  // FP8, wave 64 x 64
    {10, 64, 64, 128, 2, 2, 3, 2, 1},   // FP8, wave 32 x 32, up to 3 slots
    {11, 128, 288, 96, 4, 1, 3, 1, 2, 1},  // persistent short K: wave 32 x 288, B resident
    {12, 256, 128, 64, 2, 2, 2, 1, 2},  // wave 128 x 64: half the 256 x 256 tile's granularity
    {13, 64, 64, 128, 2, 2, 3, 2, 2},   // wave 32 x 32, 128-deep trips, up to 3 slots: small latency-bound products
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// v_mfma_f32_32x32x16_{bf16,f16} (16-bit operands) and
// v_mfma_f32_32x32x64_f8f6f4 (FP8 E4M3 operands).
constexpr int kMfmaM = 32, kMfmaN = 32, kMfmaK = 16, kMfmaK8 = 64;
constexpr int mfma_k(const TileDesc& d) { return d.esize == 1 ? kMfmaK8 : kMfmaK; }

// Epilogue band of a configuration: 32 rows x EPW columns per wave (EPW a
// multiple of 32 dividing the wave tile's width), fp32, rows padded by 16
// bytes; the bands of all waves should fit in one LDS slot (else the
// narrowest band is used and the first slot grows to hold it).
constexpr int epi_band_width(const TileDesc& d) {
  const int nw = d.wm * d.wn, wtn = d.bn / d.wn;
  const int slot = (d.bm * d.bk + d.bk * d.bn) * d.esize;
  int best = 32;
  for (int e = 32; e <= wtn; e += 32)
    if (wtn % e == 0 && nw * 32 * (e * 4 + 16) <= slot) best = e;
  return best;
}
constexpr int epi_bytes(const TileDesc& d) { return d.wm * d.wn * 32 * (epi_band_width(d) * 4 + 16); }
constexpr int slot_bytes(const TileDesc& d) { return (d.bm * d.bk + d.bk * d.bn) * d.esize; }
// LDS a kernel of this configuration declares with `stages` slots (0: the
// unstaged kernel, which holds only the epilogue bands).
constexpr int lds_bytes_for(const TileDesc& d, int stages) {
  return stages == 0 ? epi_bytes(d)
                     : (slot_bytes(d) > epi_bytes(d) ? slot_bytes(d) : epi_bytes(d)) + (stages - 1) * slot_bytes(d);
}

// Compile-time view of one configuration.
template <int ID>
struct Tile {
  static constexpr TileDesc d = kTiles[ID - 1];
  static constexpr int BM = d.bm, BN = d.bn, BK = d.bk, WM = d.wm, WN = d.wn;
  static constexpr int MAX_STAGES = d.max_stages;
  static constexpr int MIN_WAVES = d.min_waves;
  static constexpr int ES = d.esize;              // operand element bytes
  static constexpr int EPC = 16 / ES;             // elements per 16-byte chunk
  static constexpr int MK = mfma_k(d);            // k per MFMA instruction
  static constexpr int NW = WM * WN;            // waves per workgroup
  static constexpr int NT = NW * 64;            // lanes per workgroup
  static constexpr int WTM = BM / WM;           // wave tile rows
  static constexpr int WTN = BN / WN;           // wave tile columns
  static constexpr int FM = WTM / kMfmaM;       // MFMA blocks per wave along M
  static constexpr int FN = WTN / kMfmaN;       // MFMA blocks per wave along N
  static constexpr int KS = BK / MK;            // MFMA k-steps per trip
  static constexpr int CPR_A = BK * ES / 16;    // 16-byte chunks per A row (K-contiguous)
  static constexpr int CPR_B = BN * ES / 16;    // 16-byte chunks per B row (N-contiguous)
  static constexpr int CH_A = BM * CPR_A;       // chunks in one A slot
  static constexpr int CH_B = BK * CPR_B;       // chunks in one B slot
  static constexpr int IA = (CH_A + NT - 1) / NT;  // copy rounds per lane for A
  static constexpr int IB = (CH_B + NT - 1) / NT;  // copy rounds per lane for B
  static constexpr int A_BYTES = BM * BK * ES;
  static constexpr int B_BYTES = BK * BN * ES;
  static constexpr int SLOT = A_BYTES + B_BYTES;
  static constexpr int EPW = epi_band_width(d);  // epilogue band width (columns)
  static constexpr int EPI_WAVE_BYTES = 32 * (EPW * 4 + 16);
  static constexpr int EPI_BYTES = NW * EPI_WAVE_BYTES;
  static_assert(EPI_BYTES == epi_bytes(d) && SLOT == slot_bytes(d), "one layout for host and device");
  static_assert(WTM % kMfmaM == 0 && WTN % kMfmaN == 0, "wave tile must be MFMA blocks");
  static_assert(BK % MK == 0 && (BK * ES) % 16 == 0, "BK must be whole k-steps and chunks");
  static_assert((BN * ES) % 16 == 0, "BN must be whole chunks");
};

// The persistent short-K kernel (tile 11): one workgroup per CU loops over
// 128-row blocks of A and C.  B (K <= 96 rows, N <= 288 columns) is copied
// once into an LDS image that stays for the whole launch (rows 576 bytes
// apart, so the four rows a transposing fragment read touches fall on four
// different 64-byte bank ranges).  A blocks pass through a ring of three
// LDS slots (rows of 12 16-byte chunks, the chunk index XORed with
// (row / 4) mod 4 so that the 16 rows a fragment read touches fall on 16
// different bank groups).  Each wave's outputs pass through its own LDS
// band of 32 rows x 96 columns (16-bit outputs) or 32 x 32 (fp32).
namespace shortk {
constexpr int kBM = 128, kFN = 9, kNMax = 32 * kFN, kKMax = 96, kKS = kKMax / 16;
constexpr int kSlots = 3;
constexpr int kCprA = kKMax * 2 / 16;              // chunks per A row in LDS
constexpr int kSlotA = kBM * kCprA * 16;           // one A slot
constexpr int kCprB = kNMax * 2 / 16;              // chunks per B row in LDS
constexpr int kBBytes = kKMax * kCprB * 16;        // the B image
constexpr int kBandWave = 32 * (96 * 2 + 16);      // one wave's band (also holds 32 x 32 fp32)
constexpr int kLdsBytes = kBBytes + 4 * kBandWave + kSlots * kSlotA;
constexpr int kCopiesA = kBM * kCprA / 256;        // copy instructions per wave per A block
constexpr int kCopiesB = (kKMax * kCprB + 63) / 64;  // wave copy instructions for B
static_assert(kBM * kCprA % 256 == 0, "A blocks are whole copy rounds");
static_assert(32 * (32 * 4 + 16) <= kBandWave, "an fp32 band fits");
static_assert(kLdsBytes <= 163840, "fits gfx950's LDS");
}  // namespace shortk

// Largest power of two dividing n, minus one: the XOR mask that keeps a
// swizzled chunk index inside its row when a row has n chunks.
constexpr int swizzle_mask(int n) { return (n & -n) - 1; }

}  // namespace tcg
