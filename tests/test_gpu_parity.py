"""Parity of the HIP library with the fp64 oracle, on the GPU.

Each case prints what it runs before touching the GPU, so a failure names it.
Large workloads are checked at their full sizes, in the launch configuration
the benchmark times, on sampled (batch, KV head) units (and, for the 1M-token
stream, on sampled segments of the output; the state chain is always checked
whole). The oracle is exact for every slice it computes.
"""

import sys

import numpy as np
import pytest
import torch

import synth
from tests.parity import (all_units, compare_units, compare_units_pool, random_inputs,
                          tolerance)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    import compressive_memory_transformers_amd as m
    return m


def _say(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def run(lib, inp, seg_len, rule, **kw):
    res = lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"],
                      seg_len, rule, **kw)
    torch.cuda.synchronize()
    return res


def check(inp, res, seg_len, rule, units, tol, out_segments=None):
    eo, eM, ez = compare_units(inp, res, seg_len, rule, units, out_segments)
    _say(f"errors out={eo:.3e} M={eM:.3e} z={ez:.3e} (tol {tol:g})")
    assert eo <= tol and eM <= tol and ez <= tol, (eo, eM, ez)


# --- the five workloads ------------------------------------------------------

def test_tiny_fp32(lib):
    w = synth.WORKLOADS["tiny"]
    _say(f"tiny {w}")
    inp = synth.make_inputs(w, DEV)
    for rule in ("linear", "delta"):
        res = run(lib, inp, w.seg_len, rule)
        check(inp, res, w.seg_len, rule, all_units(w.B, w.Hkv), 1e-4)


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_hf_repro_bf16(lib, rule):
    w = synth.WORKLOADS["hf_repro"]
    _say(f"hf_repro {rule}")
    inp = synth.make_inputs(w, DEV)
    res = run(lib, inp, w.seg_len, rule)
    check(inp, res, w.seg_len, rule, all_units(w.B, w.Hkv), 2e-2)


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_hf_repro_shape_fp32(lib, rule):
    w = synth.WORKLOADS["hf_repro"].with_(dtype="f32")
    _say(f"hf_repro shape in fp32, {rule}")
    inp = synth.make_inputs(w, DEV)
    res = run(lib, inp, w.seg_len, rule)
    check(inp, res, w.seg_len, rule, [(0, 0), (3, 7), (7, 15)], 1e-4)


def _full_size_check(lib, w, rule, units, out_segments=None):
    """A workload at its full size in the benchmark's launch configuration
    (full workspace), inputs made on the CPU from the per-slice seeds and
    copied to the GPU; the oracle checks ``units`` in a pool of processes."""
    inp = {k: v.to(DEV) for k, v in synth.make_inputs(w, "cpu").items()}
    res = run(lib, inp, w.seg_len, rule)
    del inp
    eo, eM, ez = compare_units_pool(w, rule, res, units, out_segments=out_segments)
    _say(f"errors out={eo:.3e} M={eM:.3e} z={ez:.3e} over {len(units)} units (tol 2e-2)")
    assert eo <= 2e-2 and eM <= 2e-2 and ez <= 2e-2, (eo, eM, ez)


def test_llama3_8b_shape(lib):
    w = synth.WORKLOADS["llama3_8b"]
    _say("llama3_8b (delta, GQA 32/8), all 32 (batch, KV head) units")
    _full_size_check(lib, w, "delta", all_units(w.B, w.Hkv))


def test_long_stream(lib):
    w = synth.WORKLOADS["long_stream"]
    segs = {0, 1, 2, 127, 255, 383, 510, 511}
    _say(f"long_stream (linear, 512 segments), all 16 heads' state, out segments {sorted(segs)}")
    _full_size_check(lib, w, "linear", all_units(w.B, w.Hkv), out_segments=segs)


def test_small_segment_outliers(lib):
    w = synth.WORKLOADS["small_segment"]
    # 32 units spread over the batch and the heads (the grid's first, middle
    # and last workgroups among them)
    units = sorted({(b, (7 * b + 3 * k) % w.Hkv) for b in range(w.B) for k in range(2)})
    _say(f"small_segment (delta, 256 segments of 128, outlier keys), {len(units)} units")
    _full_size_check(lib, w, "delta", units)


# --- shapes, edge cases, and the ABI's promises -------------------------------

EDGE = [
    # B, Hq, Hkv, L, d, seg_len, dtype
    (1, 1, 1, 1, 32, 16, torch.float32),      # one token
    (1, 2, 1, 37, 32, 16, torch.float32),     # ragged last segment, GQA 2
    (2, 4, 2, 70, 64, 1, torch.float32),      # one-token segments
    (1, 3, 3, 50, 64, 200, torch.float32),    # seg_len > L
    (2, 4, 1, 300, 128, 96, torch.float32),   # GQA 4, 3 waves' worth of rows, ragged
    (1, 2, 2, 257, 128, 130, torch.bfloat16), # ragged key tiles and query tiles
    (2, 8, 2, 500, 64, 128, torch.bfloat16),
    (1, 4, 4, 64, 32, 33, torch.bfloat16),
    (1, 2, 2, 200, 128, 64, torch.bfloat16),  # direct scan (seg_len < d), bf16, d = 128
    (2, 4, 2, 90, 64, 40, torch.bfloat16),    # direct scan, GQA 2, ragged
    # seg_len >= d: the scan runs in affine form
    (1, 2, 2, 600, 32, 130, torch.float32),
    (2, 4, 2, 1100, 64, 300, torch.bfloat16),
    (1, 4, 1, 1500, 128, 520, torch.bfloat16),
    (1, 2, 2, 1200, 128, 600, torch.float32),
    # GQA blocks of four heads per position block (bf16, d in {64, 128})
    (1, 16, 2, 650, 128, 300, torch.bfloat16),  # GQA 8: two head groups per block, ragged
    (1, 8, 2, 333, 64, 333, torch.bfloat16),    # GQA 4, the last position block past the end
]


@pytest.mark.parametrize("case", EDGE, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}L{c[3]}d{c[4]}N{c[5]}{str(c[6])[6:]}" for c in EDGE])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_edge_shapes(lib, case, rule):
    B, Hq, Hkv, L, d, N, dt = case
    _say(f"edge {case} {rule}")
    inp = random_inputs(B, Hq, Hkv, L, d, dt, DEV, seed=L + d)
    res = run(lib, inp, N, rule)
    check(inp, res, N, rule, all_units(B, Hkv), tolerance(dt))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_nonzero_initial_state(lib, dt, rule):
    _say(f"nonzero M0, z0 {dt} {rule}")
    inp = random_inputs(2, 4, 2, 200, 64, dt, DEV, seed=7, m0_scale=0.5)
    res = run(lib, inp, 64, rule)
    check(inp, res, 64, rule, all_units(2, 2), tolerance(dt))


@pytest.mark.parametrize("seg_len", [100, 260])  # direct scan, affine form
def test_windows_match_one_pass(lib, seg_len):
    """A workspace of the minimum size walks the segments in windows; the
    result equals the one-pass result bit for bit."""
    _say(f"windowed vs one pass, seg_len {seg_len}")
    inp = random_inputs(2, 4, 2, 1000, 64, torch.bfloat16, DEV, seed=3)
    B, Hq, L, d = inp["q"].shape
    full, least = lib.workspace_size(B, Hq, 2, L, d, seg_len, "delta", torch.bfloat16)
    a = run(lib, inp, seg_len, "delta")
    for size in (least, least + (full - least) // 3):
        ws = torch.empty(size, dtype=torch.uint8, device=DEV)
        b = run(lib, inp, seg_len, "delta", workspace=ws)
        for x, y in zip(a, b):
            assert torch.equal(x, y)


@pytest.mark.parametrize("seg_len", [64, 256])  # direct scan, affine form
def test_in_place_state_carry(lib, seg_len):
    """M_final may be M0 and z_final may be z0."""
    _say(f"in-place carry, seg_len {seg_len}")
    inp = random_inputs(1, 4, 2, 1024, 64, torch.bfloat16, DEV, seed=5, m0_scale=0.3)
    ref = run(lib, inp, seg_len, "delta")
    M = inp["M0"].clone()
    z = inp["z0"].clone()
    res = lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], M, z, seg_len, "delta",
                      M_final=M, z_final=z)
    torch.cuda.synchronize()
    assert torch.equal(res[0], ref[0]) and torch.equal(M, ref[1]) and torch.equal(z, ref[2])


@pytest.mark.parametrize("seg_len", [64, 256])  # direct scan, affine form
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_chunked_calls_equal_one_call(lib, rule, seg_len):
    _say(f"chunked calls {rule} seg_len {seg_len}")
    inp = random_inputs(1, 2, 2, 6 * seg_len, 64, torch.float32, DEV, seed=11)
    out, M, z = run(lib, inp, seg_len, rule)
    cut = 3 * seg_len
    first = {k: (v[:, :, :cut].contiguous() if k in "qkv" else v) for k, v in inp.items()}
    second = {k: (v[:, :, cut:].contiguous() if k in "qkv" else v) for k, v in inp.items()}
    o1, M1, z1 = run(lib, first, seg_len, rule)
    second["M0"], second["z0"] = M1, z1
    o2, M2, z2 = run(lib, second, seg_len, rule)
    torch.testing.assert_close(torch.cat([o1, o2], dim=2), out, rtol=1e-5, atol=1e-6)
    torch.testing.assert_close(M2, M, rtol=1e-5, atol=1e-5)
    torch.testing.assert_close(z2, z, rtol=1e-6, atol=0)


def test_deterministic(lib):
    _say("determinism")
    inp = random_inputs(2, 8, 2, 2048, 128, torch.bfloat16, DEV, seed=9)
    a = run(lib, inp, 512, "delta")
    b = run(lib, inp, 512, "delta")
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_streams_and_null_stream(lib):
    _say("side stream")
    inp = random_inputs(1, 2, 2, 128, 32, torch.float32, DEV, seed=2)
    ref = run(lib, inp, 32, "linear")
    s = torch.cuda.Stream(DEV)
    with torch.cuda.stream(s):
        res = lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"],
                          32, "linear", stream=s)
    s.synchronize()
    for x, y in zip(ref, res):
        assert torch.equal(x, y)


def test_many_units_chain_per_unit(lib):
    """With at least as many (batch, KV head) units as CUs, the affine form's
    chain runs one workgroup per unit (bf16, d = 128, delta): parity on
    sampled units, and a one-segment-per-window workspace gives the bits of
    the full one."""
    B, Hq, Hkv, L, d, N = 4, 64, 64, 520, 128, 128  # 256 units, 5 segments, ragged
    _say(f"many units B{B} Hkv{Hkv} L{L} d{d} N{N} delta bf16")
    inp = random_inputs(B, Hq, Hkv, L, d, torch.bfloat16, DEV, seed=21, m0_scale=0.3)
    args = [inp[n] for n in ("q", "k", "v", "beta", "M0", "z0")]
    res = run(lib, inp, N, "delta")
    units = [(0, 0), (0, 63), (1, 17), (2, 40), (3, 5), (3, 63)]
    check(inp, res, N, "delta", units, tolerance(torch.bfloat16))
    _, least = lib.workspace_size(B, Hq, Hkv, L, d, N, "delta", torch.bfloat16)
    ws = torch.empty(least, dtype=torch.uint8, device=DEV)
    o2, M2, z2 = lib.forward(*args, N, "delta", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(res[0], o2) and torch.equal(res[1], M2) and torch.equal(res[2], z2)
