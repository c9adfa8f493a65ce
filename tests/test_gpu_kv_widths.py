"""Parity of the forward with a key width different from the value width
(infini_attn_forward_kv) with the fp64 oracle, on the GPU.

"Infini-Attention" (AI Wiki), "How does the compressive memory work?": the
memory maps d_key-dimensional features to d_value-dimensional values. q and
k have d_key columns, v and the output d_value, M is d_key x d_value. Every
ordered pair of distinct widths in {32, 64, 128} runs, in both element types
and both update rules, with ragged segments, grouped heads and a non-zero
initial state; whole-tensor comparison on every (batch, KV head) unit. Each
case prints what it runs before touching the GPU.
"""

import sys

import pytest
import torch

from tests.parity import all_units, compare_units, random_inputs, tolerance

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    import compressive_memory_transformers_amd as m
    return m


def _say(msg):
    print(f"[kv] {msg}", flush=True)
    sys.stdout.flush()


PAIRS = [(32, 64), (32, 128), (64, 32), (64, 128), (128, 32), (128, 64)]
CASES = [
    # B, Hq, Hkv, L, seg_len, M0 scale
    (1, 2, 2, 300, 128, 0.0),    # ragged last segment
    (2, 4, 1, 200, 64, 0.4),     # GQA 4, non-zero M0, every segment full but the last
]


@pytest.mark.parametrize("pair", PAIRS, ids=[f"dk{a}dv{b}" for a, b in PAIRS])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_kv_widths_match_the_oracle(lib, pair, dt, rule):
    dk, dv = pair
    for ci, (B, Hq, Hkv, L, N, m0) in enumerate(CASES):
        _say(f"dk={dk} dv={dv} {dt} {rule} B{B} Hq{Hq} Hkv{Hkv} L{L} N{N} m0={m0}")
        inp = random_inputs(B, Hq, Hkv, L, dk, dt, DEV, seed=dk + 3 * dv + ci, m0_scale=m0,
                            dv=dv)
        res = lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"], N,
                          rule)
        torch.cuda.synchronize()
        assert res[0].shape == (B, Hq, L, dv) and res[1].shape == (B, Hkv, dk, dv)
        eo, eM, ez = compare_units(inp, res, N, rule, all_units(B, Hkv))
        tol = tolerance(dt)
        _say(f"errors out={eo:.3e} M={eM:.3e} z={ez:.3e} (tol {tol:g})")
        assert eo <= tol and eM <= tol and ez <= tol, (eo, eM, ez)


@pytest.mark.parametrize("pair", [(64, 128), (128, 32)], ids=["dk64dv128", "dk128dv32"])
def test_kv_windows_and_in_place_carry(lib, pair):
    """The minimum workspace (one segment per window) gives the bits of the
    full one, and M_final = M0, z_final = z0 (in-place carry) gives the same
    state as separate outputs."""
    dk, dv = pair
    B, Hq, Hkv, L, N = 1, 4, 2, 500, 96
    _say(f"windows and in-place carry dk={dk} dv={dv}")
    inp = random_inputs(B, Hq, Hkv, L, dk, torch.bfloat16, DEV, seed=11, m0_scale=0.3, dv=dv)
    args = [inp[n] for n in ("q", "k", "v", "beta", "M0", "z0")]
    full, least = lib.workspace_size_kv(B, Hq, Hkv, L, dk, dv, N, "delta", torch.bfloat16)
    assert least < full
    o1, M1, z1 = lib.forward(*args, N, "delta")
    ws = torch.empty(least, dtype=torch.uint8, device=DEV)
    o2, M2, z2 = lib.forward(*args, N, "delta", workspace=ws)
    M0c, z0c = inp["M0"].clone(), inp["z0"].clone()
    o3, M3, z3 = lib.forward(*args[:4], M0c, z0c, N, "delta", M_final=M0c, z_final=z0c)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(M1, M2) and torch.equal(z1, z2)
    assert torch.equal(o1, o3) and torch.equal(M1, M3) and torch.equal(z1, z3)
    assert M3.data_ptr() == M0c.data_ptr()


def test_kv_split_workload(lib):
    """The kv_split workload at its full size (the launch configuration the
    benchmark times), checked on two sampled (batch, KV head) units."""
    import synth
    w = synth.WORKLOADS["kv_split"]
    units = [(0, 0), (3, 7)]
    _say(f"kv_split (d_key {w.d}, d_value {w.d_value}, delta, GQA 32/8), units {units}")
    inp = synth.make_inputs(w, DEV)
    res = lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"],
                      w.seg_len, "delta")
    torch.cuda.synchronize()
    eo, eM, ez = compare_units(inp, res, w.seg_len, "delta", units)
    _say(f"errors out={eo:.3e} M={eM:.3e} z={ez:.3e}")
    assert eo <= 2e-2 and eM <= 2e-2 and ez <= 2e-2, (eo, eM, ez)
