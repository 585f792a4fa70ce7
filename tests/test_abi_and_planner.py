"""Host-only checks of libtcgemm.so: it loads, exports every entry point the
headers declare, and its planner (tile, stage and grid decisions, argument
validation) behaves as specified -- no GPU needed (capabilities injected)."""
import os
import re

import pytest

import tensor_core_gemm_amd as tcg
from tensor_core_gemm_amd import BF16, EPI_NONE, EPI_RELU, F16, F32

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def declared_functions():
    names = []
    for fn in sorted(os.listdir(INCLUDE)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text,
                             re.M):
            names.append(m.group(1))
    return names


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"gemm_plan", "gemm_run", "gemm_plan_describe", "gemm_plan_destroy",
            "gemm_strerror", "tcg_probe_mfma", "tcg_probe_ds_read_tr16"} <= set(names)
    lib = tcg.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_strerror_names_every_code():
    for code in range(0, -11, -1):
        assert "unknown" not in tcg.gemm_strerror(code)
    assert "unknown" in tcg.gemm_strerror(-100)
    # every input type the planner accepts is named
    assert all(t in tcg.gemm_strerror(-2) for t in ("F16", "BF16", "FP8"))


CAPS = tcg.make_caps()


def plan(M, N, K, in_dtype=BF16, out_dtype=BF16, epi=EPI_RELU, flags=0, batch=1, tile=0,
         caps=CAPS, split_k=0, **strides):
    d = tcg.make_desc(M, N, K, in_dtype, out_dtype, epi, flags, batch,
                      strides.get("sa", 0), strides.get("sb", 0), strides.get("sc", 0), tile,
                      split_k)
    return tcg.gemm_plan_for_caps(d, caps)


def test_stage_depth_rule():
    """Page "Module Tolk.Stage", depth: 2 with async copies where two stages
    fit, 1 where one does, 0 where none does, where no tile is given, where
    a tile is below one 16-byte copy, or where staging is off."""
    caps = tcg.make_caps(lds_bytes=163840)
    slot = [32768, 32768]
    assert tcg.gemm_stage_depth(caps, 0, slot) == 2
    assert tcg.gemm_stage_depth(caps, 90000, slot) == 1       # 73840 left: one slot of 65536
    assert tcg.gemm_stage_depth(caps, 100000, slot) == 0      # 63840 left: none
    assert tcg.gemm_stage_depth(tcg.make_caps(async_copy=0), 0, slot) == 1
    assert tcg.gemm_stage_depth(caps, 0, []) == 0
    assert tcg.gemm_stage_depth(caps, 0, [8, 4096]) == 0
    assert tcg.gemm_stage_depth(caps, 0, slot, stage_enabled=False) == 0
    assert tcg.gemm_stage_depth(tcg.make_caps(lds_bytes=0), 0, slot) == 0
    assert tcg.gemm_stage_depth(tcg.make_caps(wave_size=0), 0, slot) == 0
    # exactly full
    assert tcg.gemm_stage_depth(tcg.make_caps(lds_bytes=131072), 0, [65536, 65536]) == 1
    assert tcg.gemm_stage_depth(tcg.make_caps(lds_bytes=262144), 0, [65536, 65536]) == 2


def test_headline_plan():
    p = plan(4096, 4096, 4096)
    i = p.info()
    assert (i.tile_id, i.bm, i.bn, i.bk, i.waves, i.stages) == (1, 256, 256, 64, 4, 2)
    assert i.lds_bytes == 2 * (256 * 64 + 64 * 256) * 2 == 131072
    assert (i.tiles_m, i.tiles_n, i.workgroups, i.trips) == (16, 16, 256, 64)
    # MFMA count: tiles * (256/32)^2 blocks * trips * (64/16) k-steps
    assert i.mfma_per_run == 256 * 64 * 64 * 4 == 4194304
    assert i.vec16 == 1
    assert "stages 2" in p.describe()


def test_stage_fallbacks_follow_lds_budget():
    assert plan(4096, 4096, 4096, tile=1, caps=tcg.make_caps(lds_bytes=100 * 1024)).info().stages == 1
    assert plan(4096, 4096, 4096, tile=1, caps=tcg.make_caps(lds_bytes=40 * 1024)).info().stages == 0
    assert plan(4096, 4096, 4096, tile=1, caps=tcg.make_caps(async_copy=0)).info().stages == 1
    assert plan(4096, 4096, 4096, flags=tcg.FLAG_FORCE_STAGES_1).info().stages == 1
    p = plan(4096, 4096, 4096, flags=tcg.FLAG_UNSTAGED)
    # the unstaged kernel holds only its epilogue bands: 4 waves x 32 rows x (64 fp32 + 16 B)
    assert p.info().stages == 0 and p.info().lds_bytes == 4 * 32 * (64 * 4 + 16)


def test_short_k_token_projection_takes_the_persistent_tile():
    """Many rows, K <= 96 and N <= 288 (multiples of 8), at least two 128-row
    blocks per CU: the persistent short-K kernel (tile 11), one workgroup
    per CU (grid = CUs) over ceil(M / 128) blocks, three A slots."""
    i = plan(129600, 288, 96, F16, F16, EPI_NONE).info()
    assert (i.tile_id, i.bm, i.bn, i.bk, i.stages) == (11, 128, 288, 32, 3)
    assert (i.tiles_m, i.tiles_n, i.workgroups, i.trips) == (1013, 1, 256, 3)
    assert i.lds_bytes == 96 * 576 + 4 * 32 * 208 + 3 * 128 * 192
    assert i.mfma_per_run == 1013 * 4 * 9 * 6
    assert plan(129600, 288, 96, F16, F16, EPI_RELU).info().tile_id == 11
    assert plan(65536, 192, 64, BF16, F32, EPI_NONE).info().tile_id == 11
    assert plan(65535, 192, 64, BF16, F32, EPI_NONE).info().tile_id != 11  # under two blocks per CU
    assert "persistent" in plan(129600, 288, 96, F16, F16, EPI_NONE).describe()


def test_short_k_falls_back_to_the_wide_tile():
    """Where the persistent kernel does not apply, short-K products whose N is
    a multiple of 96 take the 256 x 96 tile."""
    def tile(M=129600, N=288, K=96, **kw):
        return plan(M, N, K, F16, F16, EPI_NONE, **kw).info()
    i = tile(caps=tcg.make_caps(num_cus=1024))  # fewer blocks than CUs
    assert (i.tile_id, i.bm, i.bn, i.bk, i.tiles_n, i.trips) == (4, 256, 96, 32, 3, 3)
    assert tile(K=128).tile_id == 4
    assert tile(N=384).tile_id == 4
    assert tile(flags=tcg.FLAG_BIAS).tile_id == 4
    assert tile(flags=tcg.FLAG_UNSTAGED).tile_id == 4
    assert tile(flags=tcg.FLAG_FORCE_STAGES_1).tile_id == 4
    assert tile(flags=tcg.FLAG_FORCE_STAGES_2).tile_id == 4
    assert tile(batch=2, sa=129600 * 96, sb=96 * 288, sc=129600 * 288).tile_id == 4
    assert plan(129600, 288, 96, F16, F16, 2).info().tile_id == 4  # gelu


def test_persistent_tile_rejects_what_it_does_not_take():
    ok = dict(M=5000, N=288, K=96, in_dtype=F16, out_dtype=F16, epi=EPI_NONE, tile=11)
    assert plan(**ok).info().tile_id == 11
    for kw in (dict(K=104), dict(N=296), dict(K=92), dict(N=100), dict(M=0), dict(K=0),
               dict(batch=2, sa=5000 * 96, sb=96 * 288, sc=5000 * 288), dict(flags=tcg.FLAG_BIAS), dict(flags=tcg.FLAG_UNSTAGED),
               dict(flags=tcg.FLAG_FORCE_STAGES_1), dict(flags=tcg.FLAG_FORCE_STAGES_2),
               dict(split_k=2), dict(epi=2), dict(in_dtype=tcg.FP8)):
        with pytest.raises(tcg.GemmError) as e:
            plan(**{**ok, **kw})
        assert e.value.code == tcg.GEMM_E_ARG, kw
    with pytest.raises(tcg.GemmError) as e:
        plan(**ok, caps=tcg.make_caps(lds_bytes=128 * 1024))
    assert e.value.code == tcg.GEMM_E_DEVICE
    # fewer blocks than CUs: one workgroup per block
    assert plan(**{**ok, "M": 1000}).info().workgroups == 8


def test_ragged_and_small_shapes_fill_the_chip():
    i = plan(1000, 1000, 1000, F16, F32).info()
    assert (i.bm, i.workgroups) == (64, 256)
    i = plan(2048, 2048, 16384, BF16, BF16, EPI_NONE).info()
    assert (i.bm, i.bn, i.workgroups) == (128, 128, 256)
    i = plan(256, 256, 256, F16, F32).info()
    assert i.bm == 64


def test_deep_trip_tile_takes_unragged_one_round_grids():
    """The 64 x 64 tile with 128-deep trips: chosen where the grid gives each
    CU at most one workgroup and no tile is ragged; its third slot (one
    workgroup per CU) only past 8 trips on such a grid."""
    for M, N, K in ((1024, 1024, 1024), (512, 512, 512), (768, 768, 768), (896, 1152, 1024), (256, 256, 256)):
        i = plan(M, N, K).info()
        assert (i.tile_id, i.bk, i.stages) == (13, 128, 2), (M, N, K)
    assert plan(1000, 1000, 1000).info().tile_id == 3     # ragged edge tiles
    assert plan(1536, 1536, 1536).info().tile_id == 7     # 2.25 workgroups per CU
    assert plan(2048, 2048, 2048).info().tile_id == 7
    i = plan(512, 512, 8192).info()
    assert (i.tile_id, i.stages) == (13, 3)
    assert plan(1024, 1024, 1152).info().stages == 3     # 9 trips, one round
    assert plan(2048, 2048, 2048, tile=13).info().stages == 2   # four per CU
    assert plan(1024, 1024, 1024, tile=13).info().stages == 2   # 8 trips
    assert plan(64, 64, 8192, tile=13, split_k=8).info().stages == 2  # 8 trips per range
    assert plan(64, 64, 8192, tile=13, split_k=4).info().stages == 3
    assert plan(512, 512, 8192, tile=13, flags=tcg.FLAG_FORCE_STAGES_2).info().stages == 2


def test_vec16_needs_aligned_rows():
    assert plan(100, 64, 24).info().vec16 == 1
    assert plan(100, 64, 13).info().vec16 == 0
    assert plan(100, 60, 24).info().vec16 == 0
    assert plan(10, 16, 16, batch=2, sa=164, sb=256, sc=160).info().vec16 == 0


def test_invalid_descriptions():
    cases = [
        (dict(M=-1, N=4, K=4), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=-1), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=4, batch=0), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=4, in_dtype=F32), tcg.GEMM_E_DTYPE),
        (dict(M=4, N=4, K=4, out_dtype=9), tcg.GEMM_E_DTYPE),
        (dict(M=4, N=4, K=4, epi=7), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=4, flags=64), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=4, epi=6), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=4, epi=-1), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=4, split_k=-1), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=4, split_k=257), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=4, tile=99), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=4, batch=2, sa=15, sb=16, sc=16), tcg.GEMM_E_ARG),
        (dict(M=4, N=4, K=2**31), tcg.GEMM_E_SIZE),
    ]
    for kw, code in cases:
        with pytest.raises(tcg.GemmError) as e:
            plan(**kw)
        assert e.value.code == code, kw
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_plan_for_caps(tcg.make_desc(4, 4, 4), tcg.make_caps(wave_size=32))
    assert e.value.code == tcg.GEMM_E_DEVICE


def test_degenerate_sizes_plan():
    assert plan(0, 5, 5).info().workgroups == 0
    i = plan(5, 5, 0).info()
    assert i.trips == 0 and i.mfma_per_run == 0


FP8_TILES = (8, 9, 10)


SHORT_K_TILES = (11,)


def test_every_tile_id_plans():
    for t in range(1, tcg.gemm_tile_count() + 1):
        dt = tcg.FP8 if t in FP8_TILES else BF16
        N, K = (288, 96) if t in SHORT_K_TILES else (1000, 1000)
        i = plan(1000, N, K, in_dtype=dt, tile=t).info()
        assert i.tile_id == t and i.stages >= 2
        assert i.lds_bytes <= 163840
        # a tile is built for one operand width
        with pytest.raises(tcg.GemmError) as e:
            plan(1000, N, K, in_dtype=BF16 if t in FP8_TILES else tcg.FP8, tile=t)
        assert e.value.code == tcg.GEMM_E_ARG


def test_fp8_plans():
    """FP8 E4M3 operands: the 8-bit tiles, 64-deep MFMAs, 16-element copies."""
    i = plan(4096, 4096, 4096, in_dtype=tcg.FP8).info()
    assert (i.tile_id, i.bm, i.bn, i.bk, i.stages) == (8, 256, 256, 128, 2)
    assert i.lds_bytes == 2 * (256 * 128 + 128 * 256) == 131072
    assert (i.mfma_m, i.mfma_n, i.mfma_k) == (32, 32, 64)
    assert i.mfma_per_run == 256 * 64 * 32 * 2  # tiles x blocks x trips x k-steps
    assert i.vec16 == 1
    assert plan(4096, 4096, 4088, in_dtype=tcg.FP8).info().vec16 == 0  # K not whole 16-byte chunks
    assert plan(1000, 1000, 1000, in_dtype=tcg.FP8).info().tile_id == 10
    assert "fp8" in plan(256, 256, 256, in_dtype=tcg.FP8).describe()
    # FP8 is an operand type only
    with pytest.raises(tcg.GemmError) as e:
        plan(64, 64, 64, in_dtype=tcg.FP8, out_dtype=tcg.FP8)
    assert e.value.code == tcg.GEMM_E_DTYPE


def test_short_k_keeps_two_slots():
    """With 4 trips or fewer the ring tiles keep two slots; past that they
    take as many as fit (3 for the 64 x 64 tiles, 4 for 6 and 7)."""
    assert plan(256, 256, 256, F16, F32, tile=3).info().stages == 2   # 4 trips
    assert plan(256, 256, 320, F16, F32, tile=3).info().stages == 3   # 5 trips
    assert plan(256, 256, 512, in_dtype=tcg.FP8, tile=10).info().stages == 2
    assert plan(256, 256, 1024, in_dtype=tcg.FP8, tile=10).info().stages == 3
    assert plan(4096, 4096, 128, tile=6).info().stages == 2           # 4 trips of 32
    assert plan(4096, 4096, 4096, tile=6).info().stages == 4


def test_deep_ring_follows_lds_budget():
    """Half-depth tiles keep more chunks in flight where they fit (page
    "gizml:tile", Program.stages): 4 slots, then 3, capped at 2 on request."""
    slot = 2 * (256 * 32 + 32 * 256)
    assert plan(4096, 4096, 4096, tile=6).info().stages == 4
    assert plan(4096, 4096, 4096, tile=6, caps=tcg.make_caps(lds_bytes=3 * slot)).info().stages == 3
    assert plan(4096, 4096, 4096, tile=6, caps=tcg.make_caps(lds_bytes=2 * slot)).info().stages == 2
    assert plan(4096, 4096, 4096, tile=6, caps=tcg.make_caps(lds_bytes=2 * slot - 1)).info().stages == 1
    assert plan(4096, 4096, 4096, tile=6, flags=tcg.FLAG_FORCE_STAGES_2).info().stages == 2
    assert plan(4096, 4096, 4096, tile=6, flags=tcg.FLAG_FORCE_STAGES_1).info().stages == 1
    assert plan(4096, 4096, 4096, tile=6, caps=tcg.make_caps(async_copy=0)).info().stages == 1


def test_null_plan_is_rejected():
    fake = tcg.Plan.__new__(tcg.Plan)
    fake._h = tcg.capi._vp(None)
    fake.desc = None
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_plan_get_info(fake)
    assert e.value.code == tcg.GEMM_E_PLAN
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_run(fake, 0, 0, 0, stream=0)
    assert e.value.code == tcg.GEMM_E_PLAN


def test_gemm_plan_without_a_device_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_plan(tcg.make_desc(64, 64, 64))
    assert e.value.code == tcg.GEMM_E_DEVICE


def test_split_k_plans():
    """K cut into ranges of whole trips: workgroups, trips per range and the
    workspace follow; more ranges than trips are capped; an empty problem
    keeps one range."""
    i = plan(2048, 2048, 16384, tile=1, split_k=4).info()
    assert (i.split_k, i.trips, i.trips_per_split) == (4, 256, 64)
    assert i.workgroups == 64 * 4 and i.workspace_bytes == 4 * 2048 * 2048 * 4
    assert i.mfma_per_run == 64 * 64 * 256 * 4  # splitting adds no MFMA
    i = plan(1000, 1000, 1000, tile=3, split_k=3).info()  # 16 trips -> 6 + 6 + 4
    assert (i.split_k, i.trips_per_split) == (3, 6)
    i = plan(1000, 1000, 1000, tile=3, split_k=5).info()  # 16 trips -> 4 x 4: 4 ranges
    assert (i.split_k, i.trips_per_split) == (4, 4)
    i = plan(70, 90, 100, tile=3, split_k=8).info()
    assert (i.trips, i.split_k) == (2, 2)
    i = plan(0, 90, 100, tile=3, split_k=8).info()
    assert i.split_k == 1 and i.workspace_bytes == 0
    i = plan(70, 90, 0, tile=3, split_k=8).info()
    assert i.split_k == 1 and i.workspace_bytes == 0
    i = plan(64, 64, 4096, tile=3, split_k=2, batch=3, sa=64 * 4096, sb=4096 * 64, sc=64 * 64).info()
    assert i.workgroups == 3 * 2 and i.workspace_bytes == 2 * 3 * 64 * 64 * 4
    assert "split K 2 x 32 trips" in plan(64, 64, 4096, tile=3, split_k=2).describe()


def test_planner_splits_only_when_allowed_and_useful():
    # without the flag: never
    assert plan(128, 128, 65536).info().split_k == 1
    # with it: few output tiles and a long K are split; the square headline is not
    assert plan(128, 128, 65536, flags=tcg.FLAG_SPLIT_K).info().split_k > 1
    assert plan(512, 4096, 4096, flags=tcg.FLAG_SPLIT_K).info().split_k > 1
    i = plan(2048, 2048, 16384, flags=tcg.FLAG_SPLIT_K).info()  # measured: 134 us vs 173 unsplit
    assert (i.tile_id, i.split_k) == (1, 4)
    assert plan(4096, 4096, 4096, flags=tcg.FLAG_SPLIT_K).info().split_k == 1
    assert plan(256, 256, 256, flags=tcg.FLAG_SPLIT_K).info().split_k == 1


def test_split_tail_for_a_small_last_round():
    """With GEMM_FLAG_SPLIT_K, a problem whose tiles fill whole rounds of the
    CUs and leave a small last round runs the rows of the whole rounds
    unsplit and splits K for the rest; not where the last round is large,
    K is short, or the tile, the split or the batch is fixed."""
    S = tcg.FLAG_SPLIT_K
    i = plan(6144, 6144, 6144, flags=S).info()
    assert (i.tile_id, i.split_k, i.tail_rows, i.tail_split) == (1, 1, 768, 3)
    assert i.tiles_m == 21 and i.workgroups == 21 * 24 + 3 * 24 * 3
    assert i.workspace_bytes == 3 * 768 * 6144 * 4
    assert "last 768 rows a second launch, split K 3 x 32 trips" in plan(6144, 6144, 6144, flags=S).describe()
    i = plan(4608, 4608, 4608, flags=S).info()
    assert (i.tail_rows, i.tail_split) == (1024, 3)
    i = plan(7168, 7168, 7168, flags=S).info()
    assert (i.tail_rows, i.tail_split) == (256, 8)
    for M, N, K in ((5120, 5120, 5120), (6144, 6144, 2048), (4096, 4096, 4096), (8192, 8192, 8192)):
        assert plan(M, N, K, flags=S).info().tail_rows == 0, (M, N, K)
    assert plan(6144, 6144, 6144).info().tail_rows == 0                    # no flag
    assert plan(6144, 6144, 6144, flags=S, tile=1).info().tail_rows == 0   # tile by id
    assert plan(6144, 6144, 6144, flags=S, split_k=1).info().tail_rows == 0
    i = plan(6144, 6144, 6144, flags=S, batch=2, sa=6144 * 6144, sb=6144 * 6144, sc=6144 * 6144).info()
    assert i.tail_rows == 0
    assert plan(4096, 4096, 4096, flags=S).info().tail_split == 0
    i = plan(4608, 4608, 8192, in_dtype=tcg.FP8, flags=S).info()   # FP8: the 256 x 256 x 128 tile
    assert (i.tile_id, i.tail_rows, i.tail_split) == (8, 1024, 3)


def test_epilogue_is_named_in_the_description():
    for epi, name in ((0, "none"), (1, "relu"), (2, "gelu"), (3, "gelu_erf"), (4, "sigmoid"), (5, "tanh")):
        assert f"epilogue {name}" in plan(64, 64, 64, epi=epi).describe()
    assert "epilogue bias+tanh" in plan(64, 64, 64, epi=5, flags=tcg.FLAG_BIAS).describe()


def test_tune_cache_file_round_trip_and_tuned_plans(tmp_path):
    """A cache line names the device, the problem and the measured choice;
    gemm_plan with GEMM_FLAG_TUNED takes it, other problems keep the
    planner's choice, and a malformed file is refused."""
    tcg.gemm_tune_cache_clear()
    assert tcg.gemm_tune_cache_size() == 0
    arch = CAPS.arch.decode()
    M, N, K = 1000, 1000, 1000
    line = f"{arch} 256 {M} {N} {K} {BF16} {BF16} {EPI_RELU} {tcg.FLAG_SPLIT_K} 1 {M*K} {K*N} {M*N} 2 2 12.5\n"
    f = tmp_path / "tune.txt"
    f.write_text(line)
    tcg.gemm_tune_cache_load(str(f))
    assert tcg.gemm_tune_cache_size() == 1
    i = plan(M, N, K, flags=tcg.FLAG_SPLIT_K | tcg.FLAG_TUNED).info()
    assert (i.tile_id, i.split_k) == (2, 2)
    # the same problem without the flag, or another problem: the planner's choice
    assert plan(M, N, K, flags=tcg.FLAG_SPLIT_K).info().tile_id == 3
    assert plan(M, N, K + 8, flags=tcg.FLAG_SPLIT_K | tcg.FLAG_TUNED).info().tile_id == 3
    # a tile or split given explicitly wins over the cache
    assert plan(M, N, K, flags=tcg.FLAG_SPLIT_K | tcg.FLAG_TUNED, tile=1).info().tile_id == 1
    g = tmp_path / "saved.txt"
    tcg.gemm_tune_cache_save(str(g))
    assert g.read_text().split()[:13] == line.split()[:13]
    tcg.gemm_tune_cache_clear()
    tcg.gemm_tune_cache_load(str(g))
    assert plan(M, N, K, flags=tcg.FLAG_SPLIT_K | tcg.FLAG_TUNED).info().split_k == 2
    bad = tmp_path / "bad.txt"
    bad.write_text("gfx950 256 1 2 3\n")
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_tune_cache_load(str(bad))
    assert e.value.code == tcg.GEMM_E_ARG
    with pytest.raises(tcg.GemmError):
        tcg.gemm_tune_cache_load(str(tmp_path / "missing.txt"))
    tcg.gemm_tune_cache_clear()


def test_tuned_split_tail_entry_replays_the_planners_tail_plan(tmp_path):
    """A cache entry with split 0 stands for the planner's own plan with its
    split tail (the autotuner's extra candidate): gemm_plan with
    GEMM_FLAG_TUNED then returns that plan, tail included."""
    tcg.gemm_tune_cache_clear()
    M = N = K = 4608
    ref = plan(M, N, K, flags=tcg.FLAG_SPLIT_K).info()
    assert ref.tail_rows > 0  # this shape's last round of tiles is small
    arch = CAPS.arch.decode()
    line = (f"{arch} 256 {M} {N} {K} {BF16} {BF16} {EPI_RELU} {tcg.FLAG_SPLIT_K} 1 {M*K} {K*N} "
            f"{M*N} {ref.tile_id} 0 171.0\n")
    f = tmp_path / "tail.txt"
    f.write_text(line)
    tcg.gemm_tune_cache_load(str(f))
    i = plan(M, N, K, flags=tcg.FLAG_SPLIT_K | tcg.FLAG_TUNED).info()
    assert (i.tile_id, i.tail_rows, i.tail_split) == (ref.tile_id, ref.tail_rows, ref.tail_split)
    g = tmp_path / "saved.txt"
    tcg.gemm_tune_cache_save(str(g))
    assert g.read_text().split()[13:15] == [str(ref.tile_id), "0"]
    tcg.gemm_tune_cache_clear()


def test_run_refuses_host_tensors_before_any_launch():
    """The binding hands the kernels device addresses only: a host tensor is
    refused in Python, before the library is called (a host address would
    be written through by the GPU)."""
    import torch
    plan = tcg.gemm_plan_for_caps(tcg.make_desc(64, 64, 64, BF16, BF16, EPI_NONE), tcg.make_caps())
    A = torch.zeros(64, 64, dtype=torch.bfloat16)
    for fn in (tcg.gemm_run, tcg.gemm_run_ex, tcg.gemm_run_noalloc):
        with pytest.raises(ValueError, match="not a GPU tensor"):
            fn(plan, A, A, A, stream=0)


def test_operand_extents_follow_the_batch_strides():
    from tensor_core_gemm_amd.capi import _extent
    assert _extent(1, 0, 5, 7) == 35
    assert _extent(1, 999, 5, 7) == 35          # one item: the stride is not used
    assert _extent(3, 40, 5, 7) == 2 * 40 + 35  # the last item ends M*K past its start
    assert _extent(3, 40, 0, 7) == 0


def test_the_256_row_tile_takes_k_up_to_its_31_bit_row_offsets():
    """The 256 x 256 tile addresses row r of its A block at byte offset
    r * K * 2 inside a buffer resource of at most 2^31 - 1 bytes: K up to
    4194303 plans on it (16-byte copies up to 4194296), 4194304 is refused."""
    caps = tcg.make_caps()
    ok = tcg.gemm_plan_for_caps(tcg.make_desc(256, 64, 4194296, BF16, BF16, EPI_NONE, tile=1), caps)
    assert (ok.info().tile_id, ok.info().vec16) == (1, 1)
    ok = tcg.gemm_plan_for_caps(tcg.make_desc(256, 64, 4194303, BF16, BF16, EPI_NONE, tile=1), caps)
    assert (ok.info().tile_id, ok.info().vec16) == (1, 0)
    with pytest.raises(tcg.GemmError) as e:
        tcg.gemm_plan_for_caps(tcg.make_desc(256, 64, 4194304, BF16, BF16, EPI_NONE, tile=1), caps)
    assert e.value.code == tcg.GEMM_E_SIZE


def test_outputs_filling_one_round_of_256x128_take_that_tile():
    """16-bit operands, one batch item, K up to 4096, M a multiple of 256 and
    N of 128, the 256 x 128 grid filling between 3/4 of the CUs and all of
    them: the 256 x 128 tile (measured faster than the 128 x 128 one)."""
    for M, N, K in ((8192, 1024, 1024), (4096, 2048, 2048), (2048, 4096, 4096), (1024, 8192, 1024),
                    (7168, 1024, 512)):
        for flags in (0, tcg.FLAG_SPLIT_K):
            i = plan(M, N, K, flags=flags).info()
            assert (i.tile_id, i.workgroups, i.split_k) == (12, (M // 256) * (N // 128), 1), (M, N, K)
    # not where the grid is smaller, larger or ragged, K longer, FP8, or batched
    assert plan(2304, 2304, 2304).info().tile_id != 12       # 162 tiles: under 3/4 of the CUs
    assert plan(4608, 4608, 4608).info().tile_id != 12       # 648 tiles
    assert plan(8192, 1000, 1024).info().tile_id != 12       # ragged N
    assert plan(8192, 1024, 8192).info().tile_id != 12       # long K: left to the time model
    assert plan(8192, 1024, 1024, in_dtype=tcg.FP8).info().tile_id != 12
    assert plan(8192, 1024, 1024, batch=2, sa=8192 * 1024, sb=1024 * 1024,
                sc=8192 * 1024).info().tile_id != 12
    # a device with fewer CUs changes what one round is
    assert plan(4096, 1024, 1024, caps=tcg.make_caps(num_cus=128)).info().tile_id == 12
