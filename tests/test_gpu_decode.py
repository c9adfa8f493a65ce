"""Parity of the streaming decode step (infini_attn_decode_step) with the oracle.

A stream decoded token by token on the GPU must give the oracle forward's
output rows and, after every full segment, its state; single steps at the
Llama-3-8B shape (full 2048-row segments, 4 query heads per KV head) must
match the oracle's own decode step, including the fold of a full segment.
Each case prints what it runs before touching the GPU.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import random_inputs, tolerance

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    import compressive_memory_transformers_amd as m
    return m


def _say(msg):
    print(f"[decode] {msg}", flush=True)
    sys.stdout.flush()


def decode_stream(lib, inp, seg_len, rule):
    """Decode every token of the stream; return outputs [B,Hq,L,d] and the
    state after each full segment {tokens: (M, z)}."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    kc = torch.zeros(B, Hkv, seg_len, d, dtype=q.dtype, device=DEV)
    vc = torch.zeros_like(kc)
    M, z = inp["M0"].clone(), inp["z0"].clone()
    ws = torch.empty(lib.decode_workspace_size(B, Hq, Hkv, d, seg_len, rule, q.dtype),
                     dtype=torch.uint8, device=DEV)
    outs, states = [], {}
    for t in range(L):
        pos = t % seg_len
        o = lib.decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                            v[:, :, t].contiguous(), inp["beta"], kc, vc, M, z, pos, rule,
                            workspace=ws)
        outs.append(o)
        if pos == seg_len - 1:
            states[t + 1] = (M.clone(), z.clone())
    torch.cuda.synchronize()
    return torch.stack(outs, dim=2), states


STREAMS = [
    # B, Hq, Hkv, L, d, seg_len, dtype   (seg_len >= d folds in affine form)
    (2, 4, 2, 100, 64, 40, torch.float32),
    (2, 4, 2, 100, 64, 40, torch.bfloat16),
    (1, 8, 2, 70, 128, 32, torch.bfloat16),     # GQA 4, d = 128
    (1, 2, 1, 300, 32, 130, torch.float32),     # affine fold, ragged tail
    (1, 4, 2, 600, 32, 260, torch.bfloat16),    # affine fold, two chunks of 256 rows
    (1, 1, 1, 5, 32, 1, torch.float32),         # one-token segments
]


@pytest.mark.parametrize("case", STREAMS,
                         ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}L{c[3]}d{c[4]}N{c[5]}{str(c[6])[6:]}"
                              for c in STREAMS])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_decoded_stream_matches_the_forward(lib, case, rule):
    B, Hq, Hkv, L, d, N, dt = case
    _say(f"stream {case} {rule}")
    inp = random_inputs(B, Hq, Hkv, L, d, dt, DEV, seed=L + N, m0_scale=0.3)
    out, states = decode_stream(lib, inp, N, rule)
    f64 = {kk: synth.to_f64(vv) for kk, vv in inp.items()}
    ref, _, _ = oracle.forward(f64["q"], f64["k"], f64["v"], f64["beta"], f64["M0"], f64["z0"],
                               N, rule)
    tol = tolerance(dt)
    eo = oracle.slice_errors(synth.to_f64(out), ref)
    _say(f"out error {eo:.3e} (tol {tol:g}); {len(states)} segment ends")
    assert eo <= tol
    for n, (M, z) in states.items():
        _, M_ref, z_ref = oracle.forward(f64["q"][:, :, :n], f64["k"][:, :, :n],
                                         f64["v"][:, :, :n], f64["beta"], f64["M0"], f64["z0"],
                                         N, rule)
        eM = oracle.slice_errors(synth.to_f64(M), M_ref)
        ez = oracle.slice_errors(synth.to_f64(z), z_ref, elementwise=True)
        assert eM <= tol and ez <= tol, (n, eM, ez)


@pytest.mark.parametrize("pos", [0, 255, 256, 1000, 2047])
def test_llama_shape_steps_match_the_oracle_step(lib, pos):
    """One step at the Llama-3-8B shape (B=4, 32/8 heads, d=128, 2048-token
    segments, delta rule) with rows 0..pos-1 of the caches already filled."""
    B, Hq, Hkv, d, N, rule = 4, 32, 8, 128, 2048, "delta"
    _say(f"Llama-shape step at pos {pos}")
    g = torch.Generator(device="cpu").manual_seed(1000 + pos)
    mk = lambda *s: torch.randn(*s, generator=g, dtype=torch.float32)
    q, k, v = (mk(B, H, d).to(torch.bfloat16) for H in (Hq, Hkv, Hkv))
    kc = mk(B, Hkv, N, d).to(torch.bfloat16)
    vc = mk(B, Hkv, N, d).to(torch.bfloat16)
    beta = mk(Hq)
    M = 0.05 * mk(B, Hkv, d, d)
    z = 50.0 + torch.rand(B, Hkv, d, generator=g)
    f64 = lambda t: t.to(torch.float64).numpy()
    ro, rM, rz, rkc, _ = oracle.decode_step(f64(q), f64(k), f64(v), f64(beta), f64(M), f64(z),
                                            f64(kc), f64(vc), pos, N, rule)
    dq, dk, dv, dkc, dvc, dbeta, dM, dz = (t.to(DEV).contiguous()
                                           for t in (q, k, v, kc, vc, beta, M, z))
    out = lib.decode_step(dq, dk, dv, dbeta, dkc, dvc, dM, dz, pos, rule)
    torch.cuda.synchronize()
    eo = oracle.slice_errors(synth.to_f64(out)[:, :, None], ro[:, :, None])
    _say(f"out error {eo:.3e}")
    assert eo <= 2e-2
    assert torch.equal(dkc[:, :, pos].cpu(), k)  # the token joined the cache
    assert torch.equal(dkc[:, :, :pos].cpu(), kc[:, :, :pos])
    if pos == N - 1:
        eM = oracle.slice_errors(synth.to_f64(dM), rM)
        ez = oracle.slice_errors(synth.to_f64(dz), rz, elementwise=True)
        _say(f"fold errors M {eM:.3e} z {ez:.3e}")
        assert eM <= 2e-2 and ez <= 2e-2
    else:
        assert torch.equal(dM.cpu(), M) and torch.equal(dz.cpu(), z)


def test_decode_on_a_side_stream(lib):
    _say("side stream")
    inp = random_inputs(1, 2, 2, 8, 32, torch.float32, DEV, seed=4)
    ref, _ = decode_stream(lib, inp, 4, "delta")
    s = torch.cuda.Stream(DEV)
    with torch.cuda.stream(s):
        res, _ = decode_stream(lib, inp, 4, "delta")
    s.synchronize()
    assert torch.equal(ref, res)
