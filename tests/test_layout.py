"""The LDS layout of the staged kernels, checked on the CPU (page "Module
Tolk.Stage": global -> shared, swizzled -> fragments).

tests/layout_check.cpp evaluates the very functions the kernels use
(tensor_core_gemm_amd/csrc/tcgemm_layout.h: the swizzles, the copy plan and
the fragment-read addresses) for every tile configuration, built with g++.
For each tile this checks:
- the copy plan fills every logical chunk of the A and B tiles exactly once
  (a bijection from chunk positions to (row, chunk));
- every row's XOR stays inside the row (a per-row bijection);
- every lane's fragment read, for every wave, k-step and MFMA block, lands
  on the position holding the logical chunk the MFMA operand layout asks
  for, and the transposing reads hand each lane the column and k values it
  needs under the instruction's lane permutation (the permutation itself is
  measured on the GPU by the probe tests);
- a bank model of gfx950's LDS (64 banks of 4 bytes, 256 bytes a cycle:
  16 lanes of a 16-byte read, 32 lanes of an 8-byte read): the reads touch
  every bank once, i.e. without conflicts.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lay(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("layout") / "liblayout.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-shared", "-fPIC", "-Wall",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "tensor_core_gemm_amd", "csrc"),
                    os.path.join(ROOT, "tests", "layout_check.cpp"), "-o", out], check=True)
    lib = ctypes.CDLL(out)
    buf = (ctypes.c_int * 65536)()

    def q(tile, what, a0=0, a1=0, a2=0, a3=0):
        n = lib.layout_query(tile, what, a0, a1, a2, a3, buf)
        assert n >= 0
        return np.frombuffer(buf, dtype=np.int32, count=2 * n if what <= 1 else n).copy()

    def sk(what, a0=0, a1=0, a2=0, a3=0):
        n = lib.layout_shortk_query(what, a0, a1, a2, a3, buf)
        assert n >= 0
        return np.frombuffer(buf, dtype=np.int32, count=2 * n if what == 0 else n).copy()

    q.count = lib.layout_tile_count()
    q.shortk = sk
    return q


def tiles(lay):
    out = []
    for t in range(1, lay.count + 1):
        g = lay(t, 4)
        keys = ("ES", "CPR_A", "CPR_B", "WM", "WN", "WTM", "WTN", "MK", "BM", "BN", "BK", "persistent")
        d = dict(zip(keys, g.tolist()))
        if not d["persistent"]:  # tile 11 has its own layout (the short-K tests below)
            out.append((t, d))
    return out


def inverse_copy_map(lay, t, operand, rows, cpr):
    rc = lay(t, operand).reshape(-1, 2)
    pos = -np.ones((rows, cpr), np.int64)
    for P, (r, c) in enumerate(rc):
        pos[r, c] = P
    return pos


def test_every_configuration_is_covered(lay):
    # all but the persistent short-K tile, whose layout the short-K tests cover
    assert len(tiles(lay)) == lay.count - 1


def test_copy_plan_is_a_bijection_onto_the_tile(lay):
    for t, d in tiles(lay):
        for operand, rows, cpr in ((0, d["BM"], d["CPR_A"]), (1, d["BK"], d["CPR_B"])):
            rc = lay(t, operand).reshape(-1, 2)
            assert len(rc) == rows * cpr
            assert rc[:, 0].min() == 0 and rc[:, 0].max() == rows - 1
            assert rc[:, 1].min() == 0 and rc[:, 1].max() == cpr - 1
            flat = rc[:, 0] * cpr + rc[:, 1]
            assert np.array_equal(np.sort(flat), np.arange(rows * cpr)), (t, operand)
            # positions fill rows in order: position P lies in row P / CPR
            assert np.array_equal(rc[:, 0], np.arange(rows * cpr) // cpr)


def test_swizzle_is_a_bijection_inside_every_row(lay):
    for t, d in tiles(lay):
        for r in range(64):
            sa, sb = lay(t, 5, r)
            for cpr, x in ((d["CPR_A"], sa), (d["CPR_B"], sb)):
                assert 0 <= x < cpr
                assert sorted(c ^ x for c in range(cpr)) == list(range(cpr)), (t, r, cpr, x)


def test_a_fragment_reads_hit_their_chunks(lay):
    for t, d in tiles(lay):
        pos = inverse_copy_map(lay, t, 0, d["BM"], d["CPR_A"])
        ra = d["CPR_A"] * 16
        ks = d["BK"] // d["MK"]
        for wm in range(d["WM"]):
            wm0 = wm * d["WTM"]
            for s in range(ks):
                for lane in range(64):
                    base = int(lay(t, 2, lane, s, wm0)[0])
                    for i in range(d["WTM"] // 32):
                        off = base + i * 32 * ra
                        r = wm0 + 32 * i + (lane & 31)
                        if d["ES"] == 2:
                            wants = [(off, 2 * s + (lane >> 5))]
                        else:  # two 16-byte reads, the second at bit 4 flipped
                            wants = [(off, 4 * s + 2 * (lane >> 5)),
                                     (off ^ 16, 4 * s + 2 * (lane >> 5) + 1)]
                        for o, c in wants:
                            assert o % 16 == 0 and o // 16 == pos[r, c], (t, wm, s, lane, i)


def test_b_fragment_reads_hit_their_chunks_and_transpose(lay):
    for t, d in tiles(lay):
        pos = inverse_copy_map(lay, t, 1, d["BK"], d["CPR_B"])
        rb = d["CPR_B"] * 16
        ks = d["BK"] // d["MK"]
        es = d["ES"]
        for wn in range(d["WN"]):
            wn0 = wn * d["WTN"]
            for j in range(d["WTN"] // 32):
                for s in range(ks):
                    q = [lay(t, 3, lane, j, wn0, s) for lane in range(64)]
                    nreads = 2 if es == 2 else 4
                    for h in range(nreads):
                        # what each lane's 8-byte read covers: (row, first column)
                        cover = {}
                        for lane in range(64):
                            base, row_h0, row_h1 = (int(v) for v in q[lane])
                            step = row_h1 - row_h0  # rows between reads h and h + 1
                            off = base + (row_h0 + h * step) * rb
                            chunk, byte = divmod(off, 16)
                            r, c = divmod(int(np.argwhere(pos.ravel() == chunk)[0][0]), d["CPR_B"])
                            cover[lane] = (r, c * 16 // es + byte // es)
                        for lane in range(64):
                            g0 = lane & ~15
                            x = lane & 15
                            if es == 2:
                                # lane receives element x mod 4 of the reads of lanes 4e + x/4
                                got = [(cover[g0 + 4 * e + x // 4][0],
                                        cover[g0 + 4 * e + x // 4][1] + x % 4) for e in range(4)]
                                want = [(16 * s + 8 * (lane >> 5) + 4 * h + e, wn0 + 32 * j + (lane & 31))
                                        for e in range(4)]
                            else:
                                # lane receives byte x mod 8 of the reads of lanes 2e + x/8
                                got = [(cover[g0 + 2 * e + x // 8][0],
                                        cover[g0 + 2 * e + x // 8][1] + x % 8) for e in range(8)]
                                want = [(64 * s + 32 * (lane >> 5) + 8 * h + e, wn0 + 32 * j + (lane & 31))
                                        for e in range(8)]
                            assert got == want, (t, wn, j, s, h, lane)


def test_fragment_reads_are_free_of_bank_conflicts(lay):
    """Bank model: 64 banks of 4 bytes.  A 16-byte read serves 16 lanes a
    cycle (16 different 16-byte bank groups needed); an 8-byte transposing
    read serves 32 lanes a cycle (64 different banks needed)."""
    for t, d in tiles(lay):
        ks = d["BK"] // d["MK"]
        for wm in range(d["WM"]):
            for s in range(ks):
                offs = np.array([int(lay(t, 2, lane, s, wm * d["WTM"])[0]) for lane in range(64)])
                for g in range(4):
                    groups = (offs[16 * g:16 * g + 16] // 16) % 16
                    assert len(set(groups.tolist())) == 16, (t, "A", wm, s, g)
        rb = d["CPR_B"] * 16
        for wn in range(d["WN"]):
            for j in range(d["WTN"] // 32):
                for s in range(ks):
                    q = [lay(t, 3, lane, j, wn * d["WTN"], s) for lane in range(64)]
                    for h in range(2):
                        offs = np.array([int(v[0]) + (int(v[1]) + h * (int(v[2]) - int(v[1]))) * rb
                                         for v in q])
                        for half in range(2):
                            o = offs[32 * half:32 * half + 32]
                            banks = ((o[:, None] + np.array([0, 4])[None, :]) // 4) % 64
                            assert len(set(banks.ravel().tolist())) == 64, (t, "B", wn, j, s, h, half)


def test_a_mutated_swizzle_fails_the_bank_model(lay, tmp_path):
    """The model has teeth: with B's 8-bit XOR of 2(r mod 8) on rows of 8
    chunks (the narrow FP8 tiles' earlier swizzle), rows that share a
    256-byte line take only 4 different pair offsets."""
    def pairs_for(cpr, xor_of_row):
        banks = set()
        for r in range(8):
            line_off = (r * cpr * 16) % 256
            pair = (0 ^ xor_of_row(r)) // 2
            banks.add((line_off + 32 * pair) % 256)
        return len(banks)
    assert pairs_for(8, lambda r: (2 * (r & 7)) & 7) == 4
    assert pairs_for(8, lambda r: (2 * ((r >> 1) & 7)) & 7) == 8


# ---------------------------------------------------------------------------
# The persistent short-K tile (tile 11): an A slot of 128 rows of 12 chunks
# with the XOR (r / 4) mod 4, an unswizzled row-major B tile read with the
# transposing reads, and the fragment image that then replaces B.

def _shortk_geometry(lay):
    keys = ("BM", "CPR_A", "CPR_B", "FN", "KS", "B_BYTES", "COPIES_A", "FRAG_BYTES")
    return dict(zip(keys, lay.shortk(4).tolist()))


def _shortk_positions(lay, g):
    rc = lay.shortk(0).reshape(-1, 2)
    pos = -np.ones((g["BM"], g["CPR_A"]), np.int64)
    for P, (r, c) in enumerate(rc):
        pos[r, c] = P
    return rc, pos


def test_short_k_copy_plan_is_a_bijection_onto_the_slot(lay):
    g = _shortk_geometry(lay)
    assert g["CPR_A"] == 12 and g["BM"] * g["CPR_A"] == g["COPIES_A"] * 256  # whole copy rounds
    rc, pos = _shortk_positions(lay, g)
    n = g["BM"] * g["CPR_A"]
    assert len(rc) == n and (pos >= 0).all()
    assert np.array_equal(np.sort(rc[:, 0] * g["CPR_A"] + rc[:, 1]), np.arange(n))
    P = np.arange(n)
    assert np.array_equal(rc[:, 0], P // g["CPR_A"])  # positions fill rows in order
    # the XOR keeps every chunk inside its group of four (12 is not a power of two)
    assert np.array_equal(rc[:, 1] // 4, (P % g["CPR_A"]) // 4)


def test_short_k_a_fragment_reads_hit_their_chunks(lay):
    g = _shortk_geometry(lay)
    _, pos = _shortk_positions(lay, g)
    for w in range(4):
        for s in range(g["KS"]):
            for lane in range(64):
                off = int(lay.shortk(1, lane, s, w)[0])
                r, c = 32 * w + (lane & 31), 2 * s + (lane >> 5)
                assert off % 16 == 0 and off // 16 == pos[r, c], (w, s, lane)


def test_short_k_b_reads_transpose_into_each_lanes_column(lay):
    """B sits row-major in LDS (rows of CPR_B chunks, no swizzle).  Under
    ds_read_b64_tr_b16's lane permutation (lane x of a 16-lane group gets
    element x mod 4 of the reads of lanes 4e + x/4), lane l must receive
    column 32j + (l mod 32) at rows 16s + 8(l/32) + 4h + e, e = 0..3."""
    g = _shortk_geometry(lay)
    rb = g["CPR_B"] * 16
    for j in range(g["FN"]):
        for s in range(g["KS"]):
            for h in range(2):
                cover = {}
                for lane in range(64):
                    off = int(lay.shortk(2, lane, j, s, h)[0])
                    assert off % 8 == 0 and 0 <= off and off + 8 <= g["B_BYTES"]
                    cover[lane] = (off // rb, (off % rb) // 2)
                for lane in range(64):
                    g0, x = lane & ~15, lane & 15
                    got = [(cover[g0 + 4 * e + x // 4][0], cover[g0 + 4 * e + x // 4][1] + x % 4)
                           for e in range(4)]
                    want = [(16 * s + 8 * (lane >> 5) + 4 * h + e, 32 * j + (lane & 31)) for e in range(4)]
                    assert got == want, (j, s, h, lane)


def test_short_k_fragment_image_fills_the_b_region_exactly(lay):
    """The image is written over B in place: every fragment's 1 KiB, one
    16-byte piece per lane, and together exactly the bytes of the B tile."""
    g = _shortk_geometry(lay)
    nf = g["FN"] * g["KS"]
    offs = np.array([[int(lay.shortk(3, lane, f)[0]) for lane in range(64)] for f in range(nf)])
    assert (offs % 16 == 0).all()
    assert np.array_equal(np.sort(offs.ravel()), np.arange(0, g["B_BYTES"], 16))
    assert nf * g["FRAG_BYTES"] == g["B_BYTES"]


def test_short_k_reads_are_free_of_bank_conflicts(lay):
    """Same bank model as above: 16 lanes of a 16-byte read need 16
    different 16-byte bank groups, 32 lanes of an 8-byte read 64 banks."""
    g = _shortk_geometry(lay)
    for w in range(4):
        for s in range(g["KS"]):
            offs = np.array([int(lay.shortk(1, lane, s, w)[0]) for lane in range(64)])
            for q in range(4):
                assert len(set(((offs[16 * q:16 * q + 16] // 16) % 16).tolist())) == 16, ("A", w, s, q)
    for j in range(g["FN"]):
        for s in range(g["KS"]):
            for h in range(2):
                offs = np.array([int(lay.shortk(2, lane, j, s, h)[0]) for lane in range(64)])
                for half in range(2):
                    o = offs[32 * half:32 * half + 32]
                    banks = ((o[:, None] + np.array([0, 4])[None, :]) // 4) % 64
                    assert len(set(banks.ravel().tolist())) == 64, ("B", j, s, h, half)
    for f in range(g["FN"] * g["KS"]):
        offs = np.array([int(lay.shortk(3, lane, f)[0]) for lane in range(64)])
        for q in range(4):
            assert len(set(((offs[16 * q:16 * q + 16] // 16) % 16).tolist())) == 16, ("image", f, q)


def test_short_k_model_rejects_an_unswizzled_a_slot(lay):
    """The model has teeth here too: without the XOR, rows 192 bytes apart
    put 16 lanes' 16-byte reads on only 4 different bank groups."""
    g = _shortk_geometry(lay)
    ra = g["CPR_A"] * 16
    plain = [(r * ra + 16 * 0) // 16 % 16 for r in range(16)]
    assert len(set(plain)) == 4
    swizzled = [int(lay.shortk(1, lane, 0, 0)[0]) // 16 % 16 for lane in range(16)]
    assert len(set(swizzled)) == 16
