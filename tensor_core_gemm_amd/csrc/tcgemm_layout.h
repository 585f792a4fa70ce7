// LDS layout of a staged operand slot and the lane addresses that write and
// read it (page "Module Tolk.Stage": global -> shared, swizzled ->
// fragments).  Host and device code share these functions: the kernels use
// them to place their copies and fragment reads, and host-side checks use
// them to prove, for every tile configuration, that the swizzle is a
// bijection inside each row, that each read lands on the chunk holding the
// value it wants, and which LDS banks a wave's reads touch.
//
// A slot holds an A tile (BM rows of BK elements, K-contiguous) followed by
// a B tile (BK rows of BN elements, N-contiguous).  Each is an array of
// 16-byte chunks in row-major order, CPR chunks per row, except that chunk
// c of row r sits at position r * CPR + (c ^ swz(r)).  The copies fill the
// array in position order (lane l of round i writes position i * NT + tid,
// so each wave writes 1 KiB contiguously), which is why the XOR appears on
// the global side: position P receives the logical chunk (r, c) with
// r = P / CPR and c = (P mod CPR) ^ swz(r).
#pragma once

#include "tcgemm_tiles.h"

#if defined(__HIPCC__)
#define TCG_HD __host__ __device__
#else
#define TCG_HD
#endif

namespace tcg {

// ---------------------------------------------------------------------------
// Swizzles.  The XOR value stays below the row's power-of-two chunk group
// (swizzle_mask), so the map is a bijection inside every row.  They were
// chosen by measuring fragment-read throughput on gfx950, whose LDS serves
// 64 banks of 4 bytes: for A's 16-byte row reads, the 16 rows that 16 lanes
// read must land on 16 different 16-byte bank groups; 16 / CPR rows share a
// 256-byte line, so the XOR follows r / (16 / CPR) (r / 2 for 64-deep
// slots, r / 4 for 32-deep ones).
template <int CPR>
constexpr int swz_a_shift() {
  return CPR >= 16 ? 0 : CPR >= 8 ? 1 : CPR >= 4 ? 2 : CPR >= 2 ? 3 : 4;
}
// Rows after which swz_a repeats.
template <int CPR>
constexpr int swz_a_period() {
  return (1 << swz_a_shift<CPR>()) * (swizzle_mask(CPR) + 1);
}
template <int CPR>
TCG_HD constexpr int swz_a(int r) {
  return (r >> swz_a_shift<CPR>()) & swizzle_mask(CPR);
}
// B with 16-bit elements: a transposing 8-byte read of 32 lanes covers 4
// rows and 4 adjacent chunks of each (64 bytes), so where a row has 16
// chunks or more the XOR 4(r mod 4) gives the 4 rows 4 different 64-byte
// bank ranges; narrower rows keep 2(r mod 4).  B with 8-bit elements: a
// read of 32 lanes covers 8 rows and two adjacent chunks (a 32-byte pair)
// of each, and must put the 8 pairs on 8 different 32-byte bank ranges.
// Rows of 16 chunks or more start on a 256-byte line each, so the pair XOR
// is r mod 8; narrower rows share a line 16 / CPR at a time, so the pair
// XOR follows r / (16 / CPR), modulo the pairs a row has (tiles of 8 and 4
// chunks per row: (r / 2) mod 4 and (r / 4) mod 2).  The XOR repeats every
// 8 rows in every case.
template <int CPR>
constexpr int swz_b8_shift() {
  return CPR >= 16 ? 0 : CPR >= 8 ? 1 : CPR >= 4 ? 2 : 3;
}
template <int CPR, int ES>
TCG_HD constexpr int swz_b(int r) {
  if constexpr (ES == 2)
    return (swizzle_mask(CPR) >= 15 ? 4 * (r & 3) : 2 * (r & 3)) & swizzle_mask(CPR);
  else
    return (2 * ((r >> swz_b8_shift<CPR>()) & 7)) & swizzle_mask(CPR);
}
// Rows after which swz_b repeats.
template <int ES>
constexpr int swz_b_period() {
  return ES == 2 ? 4 : 8;
}

// ---------------------------------------------------------------------------
// Copy plan: the logical chunk that position P of a slot's A (or B) chunk
// array receives.  (The element offset of that chunk inside the tile is
// r * row_pitch + EPC * c.)
struct ChunkRC {
  int r, c;
};
template <int CPR_A>
TCG_HD constexpr ChunkRC a_chunk_at(int P) {
  const int r = P / CPR_A;
  return ChunkRC{r, (P % CPR_A) ^ swz_a<CPR_A>(r)};
}
template <int CPR_B, int ES>
TCG_HD constexpr ChunkRC b_chunk_at(int P) {
  const int r = P / CPR_B;
  return ChunkRC{r, (P % CPR_B) ^ swz_b<CPR_B, ES>(r)};
}

// ---------------------------------------------------------------------------
// Fragment reads.  MFMA operand layouts (measured by the probe kernels):
// v_mfma_f32_32x32x16_{bf16,f16}: lane l holds row (or column) l mod 32 and
// k values 8 (l / 32) .. + 7; v_mfma_f32_32x32x64_f8f6f4 with FP8: row (or
// column) l mod 32 and k = 32 (l / 32) + byte.
//
// A fragment of MFMA block i at k-step s: lane l reads row
// wm0 + 32 i + (l mod 32).  16-bit operands: one 16-byte read of logical
// chunk 2 s + l / 32.  FP8: logical chunks 4 s + 2 (l / 32) and the next
// (two reads; the XOR keeps the pair, so the second read's address is the
// first's with bit 4 flipped).  The row's swizzle depends only on l
// (wm0 and 32 i are multiples of the swizzle period), so the byte offset
// inside the A region is a_frag_base(l, s, wm0) + i * 32 * RA (+ 16 for the
// second FP8 read), with RA = BK * ES bytes per row.
template <int CPR_A, int ES>
TCG_HD constexpr int a_frag_base(int lane, int s, int wm0) {
  const int RA = CPR_A * 16;
  const int r = wm0 + (lane & 31);
  const int c = ES == 2 ? 2 * s + (lane >> 5) : 4 * s + 2 * (lane >> 5);
  return r * RA + ((c ^ swz_a<CPR_A>(r)) * 16);
}

// B fragment of MFMA block j at k-step s, 16-bit operands: column
// (l mod 32) and 8 k values 16 s + 8 (l / 32) + e, read as two transposing
// 4-value reads (h = 0, 1) with ds_read_b64_tr_b16.  That instruction works
// on groups of 16 lanes: lane x of a group receives element x mod 4 of the
// reads of lanes 4 e + x / 4, e = 0..3; so lane 4 e + q reads row e of the
// group's 4 x 16 block at columns 4 q .. 4 q + 3, and lane x receives column
// x.  The row is 16 s + 8 (l / 32) + 4 h + ((l mod 16) / 4), whose swizzle
// depends only on l, so the byte offset inside the B region is
// b_frag_base(l, j, wn0) + (16 s + 4 h) * RB, RB = BN * ES bytes per row.
//
// FP8 operands: 32 k values of column (l mod 32) in four transposing 8-byte
// reads t = 0..3 with ds_read_b64_tr_b8: lane x of a 16-lane group receives
// byte x mod 8 of the reads of lanes 2 e + x / 8, e = 0..7; so lane s' of a
// group reads row 8 t + s' / 2 (+ 32 (l / 32) + 64 s) at the 8 columns
// starting 16 ((l / 16) mod 2) + 8 (s' mod 2) of the block, and lane x
// receives column x, rows 8 t .. 8 t + 7 in order.  The byte offset is
// b_frag_base(l, j, wn0) + (64 s + 8 t) * RB.
template <int CPR_B, int ES>
TCG_HD constexpr int b_frag_base(int lane, int j, int wn0) {
  const int RB = CPR_B * 16;
  if constexpr (ES == 2) {
    const int r = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int colq = wn0 + 32 * j + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    return r * RB + (((colq >> 3) ^ swz_b<CPR_B, ES>(r)) * 16) + ((colq >> 2) & 1) * 8;
  } else {
    const int r = 32 * (lane >> 5) + ((lane & 15) >> 1);
    const int colb = wn0 + 32 * j + 16 * ((lane >> 4) & 1);  // byte column of the 16-byte chunk
    return r * RB + (((colb >> 4) ^ swz_b<CPR_B, ES>(r)) * 16) + (lane & 1) * 8;
  }
}
// Row step of the h-th (16-bit) or t-th (FP8) transposing read of k-step s.
template <int ES>
TCG_HD constexpr int b_frag_row(int s, int h) {
  return ES == 2 ? 16 * s + 4 * h : 64 * s + 8 * h;
}

// ---------------------------------------------------------------------------
// The persistent short-K tile (tile 11, 16-bit operands, K <= 96, N <= 288).
//
// An A slot holds shortk::kBM rows of shortk::kCprA = 12 chunks.  Twelve is
// not a power of two, so the XOR is bounded by the row's groups of four
// chunks: chunk c of row r sits at position c ^ ((r / 4) mod 4), which stays
// inside c's group.  Rows are 192 bytes apart, so four consecutive rows
// start on four different 64-byte ranges of a 256-byte line and the XOR
// separates the four such quads that 16 lanes of a 16-byte read cover.
TCG_HD constexpr int swz_shortk_a(int r) { return (r >> 2) & 3; }
// Copy plan: position P of an A slot receives logical chunk (r, c).
TCG_HD constexpr ChunkRC shortk_a_chunk_at(int P) {
  const int r = P / shortk::kCprA;
  return ChunkRC{r, (P % shortk::kCprA) ^ swz_shortk_a(r)};
}
// Byte offset, inside the slot, of the A fragment of k-step s for wave w:
// row 32 w + (lane mod 32), logical chunk 2 s + lane / 32 (8 k-contiguous
// values, the MFMA operand layout of the 16-bit tiles above).
TCG_HD constexpr int shortk_a_frag(int lane, int s, int w) {
  const int r = 32 * w + (lane & 31);
  return r * (shortk::kCprA * 16) + 16 * ((2 * s + (lane >> 5)) ^ swz_shortk_a(r));
}
// B is copied row-major and unswizzled (K rows of shortk::kCprB * 16 = 576
// bytes; 576 mod 256 = 64, so the four rows of a transposing read fall on
// four different 64-byte bank ranges).  Lane's transposing read h (h = 0, 1)
// of the fragment of MFMA block j at k-step s: as in b_frag_base, lane
// 4 e + q of a 16-lane group reads row e of the group's 4 x 16 block at
// columns 4 q .. 4 q + 3; the block's rows start at 16 s + 8 (lane / 32)
// + 4 h, its columns at 32 j + 16 ((lane / 16) mod 2).  The byte offset is
// shortk_b_frag_base(lane) + shortk_b_frag_step(j, s, h): the lane's part
// and a part that the unrolled loops make a constant.
TCG_HD constexpr int shortk_b_frag_base(int lane) {
  const int r = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  return r * (shortk::kCprB * 16) + 2 * col;
}
TCG_HD constexpr int shortk_b_frag_step(int j, int s, int h) {
  return (16 * s + 4 * h) * (shortk::kCprB * 16) + 2 * 32 * j;
}
// The fragment image that replaces B after those reads: fragment f (block
// j, k-step s: f = j * KS + s) is kShortkFragBytes with lane l's 16 bytes
// at shortk_image_lane(l), i.e. offset shortk_image_lane(l) + f * kShortkFragBytes.
constexpr int kShortkFragBytes = 1024;
TCG_HD constexpr int shortk_image_lane(int lane) { return lane * 16; }

}  // namespace tcg
