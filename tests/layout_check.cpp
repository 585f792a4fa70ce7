// Host-side view of the LDS layout functions (tcgemm_layout.h) for every
// tile configuration, for tests/test_layout.py.  Built with g++ (no GPU
// code): it evaluates the same functions the kernels use.
#include <stdint.h>

#include "tcgemm_layout.h"

namespace {

template <int ID>
struct TileView {
  static constexpr tcg::TileDesc d = tcg::kTiles[ID - 1];
  static constexpr int ES = d.esize, EPC = 16 / ES;
  static constexpr int CPR_A = d.bk * ES / 16, CPR_B = d.bn * ES / 16;
  static constexpr int WM = d.wm, WN = d.wn, WTM = d.bm / d.wm, WTN = d.bn / d.wn;
  static constexpr int MK = ES == 2 ? 16 : 64;
};

template <int ID>
int fill(int what, int a0, int a1, int a2, int a3, int* out) {
  using V = TileView<ID>;
  switch (what) {
    case 0: {  // A copy map: out[2P], out[2P+1] = (r, c) for P < BM * CPR_A
      const int n = V::d.bm * V::CPR_A;
      for (int P = 0; P < n; ++P) {
        const tcg::ChunkRC rc = tcg::a_chunk_at<V::CPR_A>(P);
        out[2 * P] = rc.r;
        out[2 * P + 1] = rc.c;
      }
      return n;
    }
    case 1: {  // B copy map
      const int n = V::d.bk * V::CPR_B;
      for (int P = 0; P < n; ++P) {
        const tcg::ChunkRC rc = tcg::b_chunk_at<V::CPR_B, V::ES>(P);
        out[2 * P] = rc.r;
        out[2 * P + 1] = rc.c;
      }
      return n;
    }
    case 2:  // A fragment base: lane a0, k-step a1, wave row origin a2
      out[0] = tcg::a_frag_base<V::CPR_A, V::ES>(a0, a1, a2);
      return 1;
    case 3:  // B fragment offset: lane a0, block a1, wave column origin a2, k-step a3 (read 0)
      out[0] = tcg::b_frag_base<V::CPR_B, V::ES>(a0, a1, a2);
      out[1] = tcg::b_frag_row<V::ES>(a3, 0);
      out[2] = tcg::b_frag_row<V::ES>(a3, 1);
      return 3;
    case 4:  // geometry: ES, CPR_A, CPR_B, WM, WN, WTM, WTN, MK, BM, BN, BK, persistent
      out[0] = V::ES; out[1] = V::CPR_A; out[2] = V::CPR_B; out[3] = V::WM; out[4] = V::WN;
      out[5] = V::WTM; out[6] = V::WTN; out[7] = V::MK; out[8] = V::d.bm; out[9] = V::d.bn;
      out[10] = V::d.bk; out[11] = V::d.persistent;
      return 12;
    case 5:  // swizzle values for row a0: swz_a, swz_b
      out[0] = tcg::swz_a<V::CPR_A>(a0);
      out[1] = tcg::swz_b<V::CPR_B, V::ES>(a0);
      return 2;
    default:
      return -1;
  }
}

template <int ID>
int dispatch(int id, int what, int a0, int a1, int a2, int a3, int* out) {
  if constexpr (ID > tcg::kNumTiles) {
    return -1;
  } else {
    if (id == ID) return fill<ID>(what, a0, a1, a2, a3, out);
    return dispatch<ID + 1>(id, what, a0, a1, a2, a3, out);
  }
}

}  // namespace

extern "C" int layout_tile_count(void) { return tcg::kNumTiles; }

extern "C" int layout_query(int tile, int what, int a0, int a1, int a2, int a3, int* out) {
  return dispatch<1>(tile, what, a0, a1, a2, a3, out);
}

// The persistent short-K tile's own layout (the shortk_* functions).
extern "C" int layout_shortk_query(int what, int a0, int a1, int a2, int a3, int* out) {
  namespace sk = tcg::shortk;
  switch (what) {
    case 0: {  // A copy map: out[2P], out[2P+1] = (r, c) for P < kBM * kCprA
      const int n = sk::kBM * sk::kCprA;
      for (int P = 0; P < n; ++P) {
        const tcg::ChunkRC rc = tcg::shortk_a_chunk_at(P);
        out[2 * P] = rc.r;
        out[2 * P + 1] = rc.c;
      }
      return n;
    }
    case 1:  // A fragment offset: lane a0, k-step a1, wave a2
      out[0] = tcg::shortk_a_frag(a0, a1, a2);
      return 1;
    case 2:  // B transposing read offset: lane a0, block a1, k-step a2, read a3
      out[0] = tcg::shortk_b_frag_base(a0) + tcg::shortk_b_frag_step(a1, a2, a3);
      return 1;
    case 3:  // fragment image offset: lane a0, fragment a1
      out[0] = a1 * tcg::kShortkFragBytes + tcg::shortk_image_lane(a0);
      return 1;
    case 4:  // geometry: kBM, kCprA, kCprB, kFN, kKS, kBBytes, kCopiesA, kShortkFragBytes
      out[0] = sk::kBM; out[1] = sk::kCprA; out[2] = sk::kCprB; out[3] = sk::kFN; out[4] = sk::kKS;
      out[5] = sk::kBBytes; out[6] = sk::kCopiesA; out[7] = tcg::kShortkFragBytes;
      return 8;
    default:
      return -1;
  }
}
