"""Parity of the block with its projections (infini_attn_block_forward) with
the oracle: y, M_final and z_final against oracle.block_forward on the same
bf16 inputs, read back as float64; and the projected q, k, v that the call
leaves at the head of its workspace against oracle.project_qkv, element by
element. Each case prints what it runs before touching the GPU.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# bf16 inputs; q, k, v, the gated result and y are each rounded to bf16 once
# on the GPU (relative 2^-8 at most), products accumulate in float: the
# block's own forward tolerance
TOL = 2e-2


@pytest.fixture(scope="module")
def lib():
    import compressive_memory_transformers_amd as m
    return m


def _say(msg):
    print(f"[block] {msg}", flush=True)
    sys.stdout.flush()


CASES = [
    # B, L, d_model, Hq, Hkv, d, seg_len, M0 scale
    (1, 100, 96, 4, 2, 32, 32, 0.0),       # K = 96 (3 steps), every tile ragged
    (2, 300, 512, 8, 2, 64, 128, 0.3),     # row tiles across a batch boundary
    (1, 40, 64, 2, 2, 32, 40, 0.3),        # one segment, d_model < 256
    (1, 2560, 4096, 32, 8, 128, 2048, 0.0),  # Llama-3-8B layer widths, ragged 2nd segment
]
IDS = [f"B{c[0]}L{c[1]}dm{c[2]}Hq{c[3]}Hkv{c[4]}d{c[5]}N{c[6]}" for c in CASES]


def _aligned(n):
    return (n + 255) // 256 * 256


def run_case(lib, case, rule, seed, dv=None):
    B, L, dm, Hq, Hkv, d, N, m0 = case
    dv = d if dv is None else dv
    inp = synth.make_block_inputs(B, L, dm, Hq, Hkv, d, torch.bfloat16, device=DEV, seed=seed,
                                  m0_scale=m0, z0=0.5 if m0 else 1e-6, dv=dv)
    if m0:  # a positive, non-trivial z0 beside a non-zero M0
        inp["z0"] = (0.5 + torch.rand(B, Hkv, d, generator=torch.Generator().manual_seed(seed))
                     ).to(DEV)
    nbytes = lib.block_workspace_size(B, L, dm, Hq, Hkv, d, N, rule, d_value=dv)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    y, M, z = lib.block_forward(inp["x"], inp["w_qkv"], inp["w_o"], inp["beta"], inp["M0"],
                                inp["z0"], N, rule, Hq, Hkv, workspace=ws)
    torch.cuda.synchronize()
    f = {k: synth.to_f64(v) for k, v in inp.items()}
    ry, rM, rz = oracle.block_forward(f["x"], f["w_qkv"], f["w_o"], f["beta"], f["M0"], f["z0"],
                                      N, rule, Hq, Hkv, d, dv)
    gy, gM, gz = synth.to_f64(y), synth.to_f64(M), synth.to_f64(z)
    errs = dict(
        y=max(oracle.max_rel_err(gy[b], ry[b]) for b in range(B)),
        M=oracle.slice_errors(gM, rM),
        z=oracle.slice_errors(gz, rz, elementwise=True),
    )
    # q, k, v at the head of the workspace: [B,Hq,L,d], [B,Hkv,L,d], [B,Hkv,L,dv]
    # bf16, each region rounded up to 256 bytes
    nq, nk, nv = B * Hq * L * d, B * Hkv * L * d, B * Hkv * L * dv
    raw = ws.view(torch.bfloat16)
    oq, ok = 0, _aligned(nq * 2) // 2
    ov = ok + _aligned(nk * 2) // 2
    gq = raw[oq:oq + nq].view(B, Hq, L, d)
    gk = raw[ok:ok + nk].view(B, Hkv, L, d)
    gv = raw[ov:ov + nv].view(B, Hkv, L, dv)
    pq, pk, pv = oracle.project_qkv(f["x"], f["w_qkv"], Hq, Hkv, d, dv)
    # the same split of sum_i |x_i| |w_i|: the scale of the float sum's error
    aq, ak, av = oracle.project_qkv(np.abs(f["x"]), np.abs(f["w_qkv"]), Hq, Hkv, d, dv)
    proj = 0.0
    for g, r, ra in ((gq, pq, aq), (gk, pk, ak), (gv, pv, av)):
        g = synth.to_f64(g)
        # a float sum over d_model products (error at most d_model 2^-24
        # sum |x_i w_i|, to first order), then one rounding to bf16 (at most
        # 2^-8 relative, round to nearest with 8 significant bits)
        bound = 2.0 ** -8 * (np.abs(r) + dm * 2.0 ** -24 * ra) + dm * 2.0 ** -24 * ra + 1e-30
        proj = max(proj, float(np.max(np.abs(g - r) / bound)))
    errs["proj"] = proj
    return errs


@pytest.mark.parametrize("case", CASES, ids=IDS)
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_block_matches_the_oracle(lib, case, rule):
    if case[1] > 1000 and rule == "linear":
        pytest.skip("the Llama-width case runs the delta rule only")
    _say(f"{case} {rule}")
    errs = run_case(lib, case, rule, seed=case[1] + case[2])
    _say("errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["proj"] <= 1.0, errs  # every projected element within its bound
    bad = {k: v for k, v in errs.items() if k != "proj" and not v <= TOL}
    assert not bad, (bad, TOL)


KV_PAIRS = [(32, 64), (32, 128), (64, 32), (64, 128), (128, 32), (128, 64)]


@pytest.mark.parametrize("pair", KV_PAIRS, ids=[f"dk{a}dv{b}" for a, b in KV_PAIRS])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_block_with_kv_widths_matches_the_oracle(lib, pair, rule):
    """infini_attn_block_forward_kv: query and key heads d_key wide, value
    heads and the gated result d_value wide; y, M_final, z_final and every
    projected element against the oracle, for every ordered pair of widths."""
    dk, dv = pair
    case = (2, 200, 256, 4, 2, dk, 64, 0.3)  # GQA 2, ragged last segment, 2 row tiles
    _say(f"kv widths {case} d_value {dv} {rule}")
    errs = run_case(lib, case, rule, seed=dk + 3 * dv, dv=dv)
    _say("errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["proj"] <= 1.0, errs
    bad = {k: v for k, v in errs.items() if k != "proj" and not v <= TOL}
    assert not bad, (bad, TOL)


def test_two_calls_in_a_row_reuse_the_workspace(lib):
    """A second, smaller call on the same workspace gives what a fresh call
    gives (nothing depends on what the workspace held)."""
    case = (2, 300, 512, 8, 2, 64, 128, 0.0)
    B, L, dm, Hq, Hkv, d, N, _ = case
    _say(f"workspace reuse {case}")
    big = synth.make_block_inputs(B, L, dm, Hq, Hkv, d, torch.bfloat16, device=DEV, seed=3)
    small = synth.make_block_inputs(1, 150, dm, Hq, Hkv, d, torch.bfloat16, device=DEV, seed=4)
    ws = torch.empty(lib.block_workspace_size(B, L, dm, Hq, Hkv, d, N, "delta"),
                     dtype=torch.uint8, device=DEV)
    lib.block_forward(*[big[k] for k in ("x", "w_qkv", "w_o", "beta", "M0", "z0")], N, "delta",
                      Hq, Hkv, workspace=ws)
    args = [small[k] for k in ("x", "w_qkv", "w_o", "beta", "M0", "z0")]
    y1, M1, z1 = lib.block_forward(*args, N, "delta", Hq, Hkv, workspace=ws)
    y2, M2, z2 = lib.block_forward(*args, N, "delta", Hq, Hkv)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(M1, M2) and torch.equal(z1, z2)
