"""Parity of the HIP path (through the C ABI) with the CPU oracle on the GPU.

Bars: bit-exact on integer inputs; max relative error <= 1e-2 (floor at
0.01 of an output's standard deviation) on Gaussian/uniform inputs; the
staged kernels equal the unstaged kernel bit for bit (page "Module
Tolk.Stage": staging copies values unchanged); one stage equals
two stages; repeat runs are identical; nothing outside C's M x N region is
written (page "gizml:tile", Out.put / Program.write).
"""
import numpy as np
import pytest
import torch

import gemm_workloads as gw
from gemm_workloads import BF16, EPI_NONE, EPI_RELU, F16, F32
from gpu_helpers import as_bits, as_values, check_against_oracle, check_sampled, note, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    caps = t.gemm_device_caps_query(0)
    note(f"device: {caps.arch.decode()} CUs={caps.num_cus} LDS/WG={caps.lds_bytes} "
         f"clock={caps.clock_khz} kHz")
    return t


W = gw.WORKLOADS
SMALL = ["int_fp16_256", "ragged_fp16_1000"]
BIG = ["bf16_4096_relu", "swin_proj_fp16", "deepk_bf16_2048x16384"]

# The large workloads' dtype, epilogue and input recipe at sizes the oracle
# computes in full within seconds, each spanning several tiles and a ragged
# tail in M and N, on the full-size plan's tile, split and copy path: K and
# N are multiples of 8 so the 16-byte copies run, and the tile and split are
# those the planner gives the full-size workload with split K allowed (the
# benchmark's plan).
SCALED = {
    "bf16_4096_relu": gw.custom(600, 520, 704, BF16, BF16, EPI_RELU, gw.NORMAL, seed=21,
                                name="bf16_relu_600x520x704"),
    "swin_proj_fp16": gw.custom(3000, 288, 96, F16, F16, EPI_NONE, gw.NORMAL, seed=31,
                                dist_b=gw.Dist("normal", 0.0, 96 ** -0.5), name="swin_3000"),
    "deepk_bf16_2048x16384": gw.custom(300, 264, 4096, BF16, BF16, EPI_NONE, gw.NORMAL, seed=51,
                                       name="deepk_300x264x4096"),
}


def full_size_plan(tcg, w):
    return tcg.gemm_plan(tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue,
                                       tcg.FLAG_SPLIT_K)).info()


@pytest.mark.parametrize("name", SMALL)
def test_small_workloads_full(tcg, name):
    w = W[name]
    A, B = gw.make_inputs(w)
    C, _, _ = run(tcg, A, B, w)
    check_against_oracle(w, A, B, C)


@pytest.mark.parametrize("name", BIG)
def test_scaled_workloads_full(tcg, name):
    full = full_size_plan(tcg, W[name])
    w = SCALED[name]
    A, B = gw.make_inputs(w)
    split = full.split_k if full.split_k > 1 else 0
    C, _, p = run(tcg, A, B, w, tile=full.tile_id, split_k=split)
    i = p.info()
    assert (i.tile_id, i.stages, i.vec16, i.split_k) == (full.tile_id, full.stages, full.vec16,
                                                         full.split_k)
    check_against_oracle(w, A, B, C)


@pytest.mark.parametrize("name", BIG)
def test_full_size_sampled(tcg, name):
    """Full size, the planner's launch configuration (the one the benchmark
    times), 4096 sampled outputs checked one by one."""
    w = W[name]
    A, B = gw.make_inputs(w)
    C, _, _ = run(tcg, A, B, w)
    assert np.all(np.isfinite(as_values(C)))
    check_sampled(w, A, B, C)


@pytest.mark.parametrize("tile", [4, 5, 11])
def test_swin_full_size_every_output(tcg, tile):
    """The Swin projection at full size on the three short-K tiles, every
    output checked: the last tile row is ragged (129600 = 506 x 256 + 64) and
    the B copies are partial rounds, so the wait for the first chunk must
    count the copies of the waves that issue fewer; the persistent tile runs
    four blocks per workgroup through its three-slot ring."""
    w = W["swin_proj_fp16"]
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, tile=tile)
    assert p.info().tile_id == tile
    check_against_oracle(w, A, B, C)


@pytest.mark.parametrize("name", BIG)
def test_full_size_runs_are_bitwise_stable(tcg, name):
    """Three launches of the benchmark's plan give the same bits: a missing
    wait or barrier shows up as run-to-run differences."""
    w = W[name]
    A, B = gw.make_inputs(w)
    C0, _, p = run(tcg, A, B, w)
    first = as_bits(C0)
    for _ in range(2):
        assert np.array_equal(as_bits(run(tcg, A, B, w, plan=p)[0]), first)


# The persistent short-K tile runs the MFMA sequence of the 128 x 288 x 32
# tile (one stage, unstaged and two-stage kernels of its own are not built):
# its one-stage and unstaged references are that tile's.
SAME_SEQUENCE = {11: 5}


@pytest.mark.parametrize("name", list(W))
def test_staged_equals_unstaged_bitwise(tcg, name):
    w = W[name]
    A, B = gw.make_inputs(w)
    Cs, _, ps = run(tcg, A, B, w)
    tile = SAME_SEQUENCE.get(ps.info().tile_id, ps.info().tile_id)
    Cu, _, pu = run(tcg, A, B, w, flags=tcg.FLAG_UNSTAGED, tile=tile)
    assert pu.info().stages == 0 and ps.info().stages > 0
    assert np.array_equal(as_bits(Cs), as_bits(Cu))


@pytest.mark.parametrize("name", list(W))
def test_one_stage_equals_two_stages_bitwise(tcg, name):
    w = W[name]
    A, B = gw.make_inputs(w)
    C2, _, p2 = run(tcg, A, B, w)
    tile = SAME_SEQUENCE.get(p2.info().tile_id, p2.info().tile_id)
    C1, _, p1 = run(tcg, A, B, w, flags=tcg.FLAG_FORCE_STAGES_1, tile=tile)
    assert p2.info().stages >= 2 and p1.info().stages == 1
    assert np.array_equal(as_bits(C1), as_bits(C2))


@pytest.mark.parametrize("tile", [6, 7])
def test_ring_depths_give_the_same_bits(tcg, tile):
    """Rings of 4, 3 and 2 slots, one stage and no staging: one MFMA
    sequence, so the same bits (odd and even trip counts, ragged edges)."""
    for K in (1000, 992, 96):
        w = gw.custom(520, 300, K, BF16, BF16, EPI_RELU, gw.NORMAL, seed=K)
        A, B = gw.make_inputs(w)
        desc = tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, tile=tile)
        ref = None
        deep = tcg.make_desc(w.M, w.N, 1000, w.in_dtype, w.out_dtype, w.epilogue, tile=tile)
        slot = tcg.gemm_plan_for_caps(deep, tcg.make_caps()).info().lds_bytes // 4  # a 4-slot plan
        for lds, flags, want in ((163840, 0, 4), (slot * 7 // 2, 0, 3),
                                 (163840, tcg.FLAG_FORCE_STAGES_2, 2),
                                 (163840, tcg.FLAG_FORCE_STAGES_1, 1), (163840, tcg.FLAG_UNSTAGED, 0)):
            d = tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, flags, tile=tile)
            p = tcg.gemm_plan_for_caps(d, tcg.make_caps(lds_bytes=lds))
            # 4 trips or fewer keep two slots
            assert p.info().stages == (min(want, 2) if -(-K // 32) <= 4 else want)
            bits = as_bits(run(tcg, A, B, w, plan=p)[0])
            if ref is None:
                ref = bits
                check_against_oracle(w, A, B, run(tcg, A, B, w, plan=p)[0])
            assert np.array_equal(bits, ref), (K, want)
        del desc


@pytest.mark.parametrize("tile,in_dtype", [(3, F16), (3, BF16), (10, gw.FP8)])
def test_small_tile_rings_give_the_same_bits(tcg, tile, in_dtype):
    """The 64 x 64 tiles keep up to three chunks in flight: rings of 3 and 2
    slots, one stage and no staging give the same bits (ragged edges, odd
    and even trip counts, a K tail inside the last chunk)."""
    for M, N, K in ((1000, 1000, 1000), (130, 70, 448), (64, 64, 328), (300, 200, 4000)):
        w = gw.custom(M, N, K, in_dtype, F32, EPI_RELU, gw.NORMAL, seed=K + tile)
        A, B = gw.make_inputs(w)
        ref = None
        for lds, flags, want in ((163840, 0, 3), (163840, tcg.FLAG_FORCE_STAGES_2, 2),
                                 (163840, tcg.FLAG_FORCE_STAGES_1, 1), (163840, tcg.FLAG_UNSTAGED, 0)):
            d = tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, flags, tile=tile)
            p = tcg.gemm_plan_for_caps(d, tcg.make_caps(lds_bytes=lds))
            bk = 64 if tile == 3 else 128
            # 4 trips or fewer keep two slots
            assert p.info().stages == (min(want, 2) if -(-K // bk) <= 4 else want)
            C = run(tcg, A, B, w, plan=p)[0]
            if ref is None:
                ref = as_bits(C)
                check_against_oracle(w, A, B, C)
            assert np.array_equal(as_bits(C), ref), (M, N, K, want)


@pytest.mark.parametrize("in_dtype", [F16, BF16])
def test_deep_trip_tile_rings_give_the_same_bits(tcg, in_dtype):
    """The 64 x 64 tile with 128-deep trips takes three slots only for more
    than 8 trips on a grid of at most one workgroup per CU; every ring depth,
    one stage and no staging give the same bits (ragged edges, K tails)."""
    for M, N, K, deep in ((1000, 1000, 1000, False), (130, 70, 1400, True), (64, 64, 1032, True),
                          (300, 200, 4000, True), (2048, 1024, 1152, False)):
        w = gw.custom(M, N, K, in_dtype, F32, EPI_RELU, gw.NORMAL, seed=K + M)
        A, B = gw.make_inputs(w)
        ref = None
        for flags, want in ((0, 3 if deep else 2), (tcg.FLAG_FORCE_STAGES_2, 2), (tcg.FLAG_FORCE_STAGES_1, 1),
                            (tcg.FLAG_UNSTAGED, 0)):
            d = tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, flags, tile=13)
            p = tcg.gemm_plan_for_caps(d, tcg.make_caps())
            assert p.info().stages == want, (M, N, K, flags)
            C = run(tcg, A, B, w, plan=p)[0]
            if ref is None:
                ref = as_bits(C)
                check_against_oracle(w, A, B, C)
            assert np.array_equal(as_bits(C), ref), (M, N, K, want)


def test_repeat_runs_identical(tcg):
    w = W["ragged_fp16_1000"]
    A, B = gw.make_inputs(w)
    first = as_bits(run(tcg, A, B, w)[0])
    for _ in range(3):
        assert np.array_equal(as_bits(run(tcg, A, B, w)[0]), first)


@pytest.mark.parametrize("out_dtype", [F32, F16, BF16])
def test_guard_band_untouched(tcg, out_dtype):
    w = gw.custom(333, 250, 190, F16, out_dtype, EPI_RELU, gw.UNIT, seed=7)
    A, B = gw.make_inputs(w)
    guard = 4096
    sentinel = 0x5A5A5A5A if out_dtype == F32 else 0x5A5A
    C, buf, _ = run(tcg, A, B, w, guard=guard, sentinel=sentinel)
    raw = as_bits(buf)
    sent = np.array(sentinel, raw.dtype)
    assert np.all(raw[:guard] == sent) and np.all(raw[-guard:] == sent)
    check_against_oracle(w, A, B, C)


def test_batch_strides(tcg):
    w = gw.custom(130, 70, 90, BF16, F32, EPI_RELU, gw.NORMAL, seed=9, batch=3)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w)
    assert p.info().workgroups == p.info().tiles_m * p.info().tiles_n * 3
    check_against_oracle(w, A, B, C)


@pytest.mark.parametrize("tile", [1, 2, 3, 4, 5, 6, 7, 12, 13])
def test_every_tile_gives_the_exact_integer_result(tcg, tile):
    """Every tile configuration computes the same result (page "gizml:tile",
    tune requires all configurations to agree)."""
    w = gw.custom(300, 288, 300, F16, F32, EPI_NONE, gw.INT4, seed=11)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, tile=tile)
    assert p.info().tile_id == tile
    check_against_oracle(w, A, B, C)


# Trip counts around the copy schedule's boundaries: a ring of S slots runs
# the hand-interleaved trips only while chunk t + 2S exists, and then splits
# each chunk's copies between two trips; the last trips issue whole chunks
# and finish a split one.  K = BK * trips - 8 leaves a partial last chunk.
TRIP_CASES = [(tile, trips, flags) for tile, flags in ((1, 0), (2, 0), (3, 0), (6, 0), (7, 0), (12, 0), (13, 0),
                                                       (3, "stages2"), (6, "stages2"), (7, "stages2"),
                                                       (13, "stages2"))
              for trips in range(1, 10)]


@pytest.mark.parametrize("tile,trips,flags", TRIP_CASES)
def test_trip_counts_across_the_copy_schedule(tcg, tile, trips, flags):
    bk = {13: 128, 1: 64, 2: 64, 3: 64, 12: 64}.get(tile, 32)
    K = bk * trips - 8
    f = tcg.FLAG_FORCE_STAGES_2 if flags == "stages2" else 0
    w = gw.custom(300, 264, K, F16, F32, EPI_RELU, gw.INT4, seed=100 * tile + trips)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w, tile=tile, flags=f)
    info = p.info()
    assert info.tile_id == tile and info.trips == trips
    if flags == "stages2":
        assert info.stages == 2
    check_against_oracle(w, A, B, C)


EDGE = [(1, 1, 1), (1, 300, 17), (300, 1, 64), (33, 65, 16), (64, 64, 64), (257, 255, 129),
        (17, 513, 1000), (96, 96, 8)]


@pytest.mark.parametrize("M,N,K", EDGE)
@pytest.mark.parametrize("in_dtype,out_dtype", [(F16, F32), (BF16, BF16), (F16, F16)])
def test_edge_shapes(tcg, M, N, K, in_dtype, out_dtype):
    for dist in (gw.INT4, gw.NORMAL):
        w = gw.custom(M, N, K, in_dtype, out_dtype, EPI_RELU, dist, seed=M + N + K)
        A, B = gw.make_inputs(w)
        C, _, _ = run(tcg, A, B, w)
        check_against_oracle(w, A, B, C)


def test_k_zero_writes_positive_zero(tcg):
    for out_dtype in (F32, F16, BF16):
        w = gw.custom(70, 90, 0, BF16, out_dtype, EPI_NONE, gw.NORMAL)
        A = torch.zeros(0, dtype=torch.bfloat16)
        B = torch.zeros(0, dtype=torch.bfloat16)
        C, _, _ = run(tcg, A, B, w, sentinel=0x1234)
        assert np.all(as_bits(C) == 0)


@pytest.mark.parametrize("M,N,K", [(45, 21, 13), (130, 77, 250), (64, 100, 9)])
def test_element_copy_path(tcg, M, N, K):
    """K or N not a multiple of 8: rows are not 16-byte aligned, so the
    element-copy kernels run; compared with the oracle and the unstaged kernel."""
    w = gw.custom(M, N, K, F16, F32, EPI_RELU, gw.NORMAL, seed=K)
    A, B = gw.make_inputs(w)
    C, _, p = run(tcg, A, B, w)
    assert p.info().vec16 == 0
    check_against_oracle(w, A, B, C)
    Cu, _, _ = run(tcg, A, B, w, flags=tcg.FLAG_UNSTAGED, tile=p.info().tile_id)
    assert np.array_equal(as_bits(C), as_bits(Cu))


def test_misaligned_pointers_take_the_element_path(tcg):
    w = gw.custom(200, 136, 128, BF16, BF16, EPI_RELU, gw.NORMAL, seed=3)
    A, B = gw.make_inputs(w)
    C0, _, p = run(tcg, A, B, w)
    C1, _, _ = run(tcg, A, B, w, plan=p, a_offset=1, b_offset=3)
    assert np.array_equal(as_bits(C0), as_bits(C1))
    check_against_oracle(w, A, B, C0)


def test_lds_budget_fallbacks_give_the_same_bits(tcg):
    """The stage rule (page "Module Tolk.Stage", depth): with less LDS the
    planner takes one stage, then none; every plan returns the same bits."""
    w = gw.custom(512, 512, 512, BF16, BF16, EPI_RELU, gw.NORMAL, seed=5)
    A, B = gw.make_inputs(w)
    desc = tcg.make_desc(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.epilogue, tile=1)
    results = []
    for lds, want in ((163840, 2), (100 * 1024, 1), (40 * 1024, 0)):
        p = tcg.gemm_plan_for_caps(desc, tcg.make_caps(lds_bytes=lds))
        assert p.info().stages == want
        results.append(as_bits(run(tcg, A, B, w, plan=p)[0]))
    assert np.array_equal(results[0], results[1]) and np.array_equal(results[0], results[2])


def test_run_errors(tcg):
    w = gw.custom(64, 64, 64, F16, F16, EPI_NONE, gw.NORMAL)
    p = tcg.gemm_plan(tcg.make_desc(64, 64, 64, F16, F16))
    buf = torch.zeros(3 * 64 * 64, dtype=torch.float16, device="cuda")
    A, B = buf[:4096], buf[4096:8192]
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_run(p, A, B, buf[2048:6144])  # C overlaps A and B
    assert e.value.code == tcg.GEMM_E_ALIAS
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_run(p, A, B, 0)
    assert e.value.code == tcg.GEMM_E_ARG
    tcg.gemm_run(p, A, B, buf[8192:])  # disjoint: fine
    torch.cuda.synchronize()
    del w
