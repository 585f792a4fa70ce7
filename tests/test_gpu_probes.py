"""Hardware lane layouts the GEMM kernels rely on, measured on gfx950.

The fragment loaders assume (a) MFMA operand/result lane layouts, (b) the
lane permutation of the transposing LDS read ds_read_b64_tr_b16 and (c) the
LDS placement and out-of-range zero-fill of a buffer load that writes LDS
directly.  Each test runs one small in-bounds probe kernel and checks the
assumption; on a mismatch it prints what the hardware did.
"""
import json
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

# Where to keep what the probes measured (for reading after a failure): a
# directory named by TCGEMM_PROBE_OUT, if set.
OUT_DIR = os.environ.get("TCGEMM_PROBE_OUT", "")


def _record(name, obj):
    if OUT_DIR and os.path.isdir(OUT_DIR):
        with open(os.path.join(OUT_DIR, f"probe_{name}.json"), "w") as f:
            json.dump(obj, f)


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tensor_core_gemm_amd import probe as p
    return p


def _bits(x, bf16):
    t = torch.tensor(np.asarray(x, np.float32))
    t = t.to(torch.bfloat16 if bf16 else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_32x32x16_layout(probe, kind):
    """A lane l: row l%32, k 8*(l//32)+e; B lane l: col l%32, same k;
    D lane l, register r: row 8*(r//4) + 4*(l//32) + r%4, col l%32."""
    rng = np.random.default_rng(kind)
    A = rng.integers(-4, 5, (32, 16)).astype(np.float32)
    B = rng.integers(-4, 5, (16, 32)).astype(np.float32)
    bf16 = kind == 0
    a_regs = np.zeros((64, 8), np.float32)
    b_regs = np.zeros((64, 8), np.float32)
    for l in range(64):
        for e in range(8):
            a_regs[l, e] = A[l % 32, 8 * (l // 32) + e]
            b_regs[l, e] = B[8 * (l // 32) + e, l % 32]
    d = probe.mfma(kind, _bits(a_regs, bf16), _bits(b_regs, bf16))
    ref = A @ B
    want = np.zeros((64, 16), np.float32)
    for l in range(64):
        for r in range(16):
            want[l, r] = ref[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32]
    if not np.array_equal(d, want):
        _record(f"mfma32_{kind}", {"A": A.tolist(), "B": B.tolist(), "d": d.tolist()})
    assert np.array_equal(d, want)


@pytest.mark.parametrize("kind", [2, 3])
def test_mfma_16x16x32_layout(probe, kind):
    """A lane l: row l%16, k 8*(l//16)+e; D lane l, register r: row
    4*(l//16) + r, col l%16."""
    rng = np.random.default_rng(kind)
    A = rng.integers(-4, 5, (16, 32)).astype(np.float32)
    B = rng.integers(-4, 5, (32, 16)).astype(np.float32)
    bf16 = kind == 2
    a_regs = np.zeros((64, 8), np.float32)
    b_regs = np.zeros((64, 8), np.float32)
    for l in range(64):
        for e in range(8):
            a_regs[l, e] = A[l % 16, 8 * (l // 16) + e]
            b_regs[l, e] = B[8 * (l // 16) + e, l % 16]
    d = probe.mfma(kind, _bits(a_regs, bf16), _bits(b_regs, bf16))
    ref = A @ B
    want = np.zeros((64, 16), np.float32)
    for l in range(64):
        for r in range(4):
            want[l, r] = ref[4 * (l // 16) + r, l % 16]
    if not np.array_equal(d, want):
        _record(f"mfma16_{kind}", {"A": A.tolist(), "B": B.tolist(), "d": d.tolist()})
    assert np.array_equal(d, want)


def test_ds_read_tr16_permutation(probe):
    """Lane l reads 4 16-bit values at byte l*8 (value = element index), so
    source (lane s, element e) carries 4*s + e.  Measured on gfx950: within
    each group of 16 lanes, dst(lane x, element e) = src(lane 4*e + x//4,
    element x%4); the B-fragment loader's addresses are derived from it."""
    init = np.arange(4096, dtype=np.uint16)
    addr = np.arange(64, dtype=np.uint32) * 8
    out = probe.ds_read_tr16(init, addr)
    src_lane, src_elem = out // 4, out % 4
    _record("tr16", {"out": out.tolist()})
    print("dst -> (src lane, src elem):")
    for j in range(64):
        print(j, list(zip(src_lane[j].tolist(), src_elem[j].tolist())))
    want = np.zeros((64, 4), np.int64)
    for j in range(64):
        for e in range(4):
            g, x = 16 * (j // 16), j % 16
            want[j, e] = 4 * (g + 4 * e + x // 4) + x % 4
    assert np.array_equal(out.astype(np.int64), want)


def test_buffer_lds_placement_and_zero_fill(probe):
    """Lane l's 16 bytes land at LDS base + 16*l; offsets at or past
    num_records read 0 (the source allocation is twice num_records, so the
    out-of-range offsets used here still point at owned memory)."""
    words = 4096
    src = torch.arange(words, dtype=torch.int32, device="cuda") + 1000
    records = 8192  # bytes: half the allocation
    voff = np.array([((l * 37) % 64) * 16 for l in range(64)], np.uint32)
    oob = np.arange(56, 64)
    voff[oob] = 8192 + 16 * np.arange(8)  # past num_records, inside the allocation
    base = 1024
    lds = probe.buffer_lds(src, records, voff, base)
    want = np.full(2048, 0xDEADBEEF, np.uint64)
    for l in range(64):
        for w in range(4):
            v = 0 if l in oob else 1000 + voff[l] // 4 + w
            want[base // 4 + 4 * l + w] = v
    if not np.array_equal(lds.astype(np.uint64), want):
        _record("buffer_lds", {"lds": lds.tolist(), "voff": voff.tolist()})
    assert np.array_equal(lds.astype(np.uint64), want)


def test_buffer_lds_high_offset_reads_zero(probe):
    """The kernels mark masked lanes with byte offset 0x80000000; the same
    range check as above must turn it into a zero read."""
    src = torch.arange(4096, dtype=torch.int32, device="cuda") + 1000
    voff = np.array([16 * l for l in range(64)], np.uint32)
    voff[5] = 0x80000000
    voff[63] = 0x80000000
    lds = probe.buffer_lds(src, 8192, voff, 0)
    got = lds[:256].reshape(64, 4)
    for l in range(64):
        if l in (5, 63):
            assert np.all(got[l] == 0)
        else:
            assert np.array_equal(got[l], 1000 + 4 * l + np.arange(4))


def _e4m3(x):
    """FP8 E4M3 (OCP: bias 7, no infinities) patterns of exactly representable values."""
    t = torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


# Candidate maps (half h = lane // 32, register byte j) -> k of the 64-deep
# FP8 MFMA operands; the test names the one the hardware follows.
F8_K_MAPS = {
    "contiguous": lambda h, j: 32 * h + j,
    "halves_of_16": lambda h, j: 16 * h + (j % 16) + 32 * (j // 16),
    "quarters_of_8": lambda h, j: 8 * h + (j % 8) + 16 * (j // 8),
}


def test_mfma_f8_32x32x64_layout(probe):
    """Which k each operand byte holds, for v_mfma_f32_32x32x64_f8f6f4 with
    E4M3 operands: A lane l holds row l%32, B lane l column l%32, and D has
    the bf16 32x32 layout; the k of byte j of lane l is one of F8_K_MAPS."""
    rng = np.random.default_rng(5)
    A = rng.integers(-4, 5, (32, 64)).astype(np.float32)
    B = rng.integers(-4, 5, (64, 32)).astype(np.float32)
    ref = A @ B
    want = np.zeros((64, 16), np.float32)
    for l in range(64):
        for r in range(16):
            want[l, r] = ref[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32]
    found = []
    for name, kmap in F8_K_MAPS.items():
        a_regs = np.zeros((64, 32), np.float32)
        b_regs = np.zeros((64, 32), np.float32)
        for l in range(64):
            for j in range(32):
                k = kmap(l // 32, j)
                a_regs[l, j] = A[l % 32, k]
                b_regs[l, j] = B[k, l % 32]
        d = probe.mfma_f8(_e4m3(a_regs), _e4m3(b_regs))
        _record(f"mfma_f8_{name}", {"d": d.tolist(), "want": want.tolist()})
        if np.array_equal(d, want):
            found.append(name)
    print("FP8 k maps matching the hardware:", found)
    # Every consistent map gives A.B: the MFMA pairs byte j of A lane l with
    # byte j of B lane l' (l, l' in the same half), so only the pairing
    # matters, and the kernels use the contiguous one.  The exact products
    # of E4M3 integers also confirm the OCP encoding (bias 7).
    assert found == list(F8_K_MAPS)


def test_ds_read_tr8_permutation(probe):
    """Lane l reads 8 bytes at byte 8l.  Two fills name the source of every
    returned byte: one with the source lane (byte i holds i // 8), one with
    the source byte (i % 8).  Within each group of 16 lanes, lane x receives
    byte x%8 of the reads of lanes 2e + x//8, e = 0..7."""
    addr = np.arange(64, dtype=np.uint32) * 8
    idx = np.arange(512)
    lane_of = probe.ds_read_tr8((idx // 8).astype(np.uint8), addr)
    byte_of = probe.ds_read_tr8((idx % 8).astype(np.uint8), addr)
    _record("tr8", {"lane": lane_of.tolist(), "byte": byte_of.tolist()})
    print("dst -> (src lane, src byte):")
    for j in range(64):
        print(j, list(zip(lane_of[j].tolist(), byte_of[j].tolist())))
    # measured on gfx950: within each group of 16 lanes, dst(lane x, byte e)
    # = src(lane 2e + x//8, byte x%8); the FP8 B-fragment loader relies on it
    want_lane = np.zeros((64, 8), np.int64)
    want_byte = np.zeros((64, 8), np.int64)
    for j in range(64):
        g, x = 16 * (j // 16), j % 16
        for e in range(8):
            want_lane[j, e] = g + 2 * e + x // 8
            want_byte[j, e] = x % 8
    assert np.array_equal(lane_of.astype(np.int64), want_lane)
    assert np.array_equal(byte_of.astype(np.int64), want_byte)


def test_clock_probe_reports_every_xcd_and_a_plausible_clock(probe):
    """The clock probe: XCD ids within the device's count, both counters
    advance between two marks, and over a stretch of back-to-back MFMA work
    on every CU (no idle time between the marks: the shader-clock counter
    slows down with the clock when the GPU idles) the clock lies between
    500 MHz and the device's peak clock (plus margin)."""
    import tensor_core_gemm_amd as tcg
    caps = tcg.gemm_device_caps_query(0)
    wg = caps.num_cus
    ops = torch.zeros(16 * 64 * 8, dtype=torch.int16, device="cuda")
    sink = torch.empty(wg * 256, device="cuda")
    ticks = torch.zeros(wg, dtype=torch.int64, device="cuda")
    cp = probe.ClockProbe(workgroups=1024)
    torch.cuda.synchronize()
    cp.mark(0)
    for _ in range(20):
        probe.mfma_rate(probe.MFMA_32x32x16_BF16, wg, 200, ops, sink, ticks)
    cp.mark(1)
    torch.cuda.synchronize()
    a = cp.bufs[0].cpu().numpy().reshape(-1, 3)
    assert set(a[:, 0].tolist()) <= set(range(max(caps.num_xcds, 1)))
    r = cp.result()
    print(f"clock probe: {r}", flush=True)
    assert len(r["per_xcd_mhz"]) == max(caps.num_xcds, 1)
    assert 500 <= r["min_mhz"] and r["max_mhz"] <= caps.clock_khz / 1000 * 1.1
    assert r["seconds"] > 0


def test_mfma_rate_probe_issues_back_to_back(probe):
    """The register-only MFMA loop: every workgroup's loop takes about 32
    shader cycles per v_mfma_f32_32x32x16_bf16 (8 passes of 4 cycles, the
    rate the dense peak assumes), and its outputs are finite."""
    wg, iters = 64, 10
    gen = torch.Generator().manual_seed(3)
    ops = (torch.randn(16 * 64 * 8, generator=gen) * 0.01).to(torch.bfloat16).view(torch.int16).cuda()
    sink = torch.full((wg * 256,), float("nan"), device="cuda")
    ticks = torch.zeros(wg, dtype=torch.int64, device="cuda")
    flops = probe.mfma_rate(probe.MFMA_32x32x16_BF16, wg, iters, ops, sink, ticks)
    torch.cuda.synchronize()
    assert flops == wg * 4 * iters * 64 * 32768
    assert torch.isfinite(sink).all()
    cyc = ticks.cpu().numpy() / (iters * 64)
    print(f"cycles per MFMA: median {np.median(cyc):.2f}", flush=True)
    assert np.all(cyc >= 31.5) and np.median(cyc) <= 40


def test_copy_issue_probe_runs_every_pattern(probe):
    """The copy-issue probe: every pattern runs; without copies the loop
    issues an MFMA every ~32 cycles per SIMD with one or two waves, and
    copies never make it faster."""
    import tensor_core_gemm_amd as tcg
    wg = 32
    ops = (torch.randn(8 * 64 * 8) * 0.01).to(torch.bfloat16).view(torch.int16).cuda()
    src = torch.zeros(65536 // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(wg * 512, device="cuda")
    ticks = torch.zeros(wg, dtype=torch.int64, device="cuda")
    got = {}
    for pat in probe.COPY_PATTERNS:
        per_simd = probe.copy_issue(pat, wg, 20, ops, src, sink, ticks)
        torch.cuda.synchronize()
        got[pat] = float(np.median(ticks.cpu().numpy())) / per_simd
        assert torch.isfinite(sink[: wg * 256]).all()
    print(f"cycles per MFMA per SIMD: {got}", flush=True)
    assert 31.5 <= got[0] <= 40 and 31.5 <= got[3] <= 40
    assert got[1] >= got[0] * 0.98 and got[4] >= got[3] * 0.98
    # the 16x16x32 shape: half the cycles of an MFMA at the peak rate
    assert 15.5 <= got[6] <= 24 and got[7] >= got[6] * 0.98
    with pytest.raises(RuntimeError):
        probe.copy_issue(99, wg, 1, ops, src, sink, ticks)
