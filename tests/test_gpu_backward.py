"""Parity of the backward pass (infini_attn_backward) and of the training
forward's softmax statistics (infini_attn_forward_train) with the oracle.

The GPU gradients of the loss sum(d_out*out) + sum(dM_final*M_final) +
sum(dz_final*z_final) are compared, per (batch, head) slice and normwise, with
oracle.backward on the same (rounded) inputs; lse with the base-2
log-sum-exp of the scaled scores computed in float64. Each case prints what
it runs before touching the GPU.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# float: every product in float, the error is rounding in the order of
# summation (seen: 1e-5 or less); bf16: the products take bf16 operands
# (sigma(Q), dn, M_{s-1}, dM_s, U, dP, and the bf16 inputs) with float
# accumulation, relative rounding 2^-9 per operand, a few in a row (seen:
# 1.1e-2 or less, the largest for one-token segments, where dQ is the small
# retrieval part alone); the dM recurrence itself runs in float
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def lib():
    import compressive_memory_transformers_amd as m
    return m


def _say(msg):
    print(f"[backward] {msg}", flush=True)
    sys.stdout.flush()


CASES = [
    # B, Hq, Hkv, L, d, seg_len, dtype
    (1, 2, 1, 40, 32, 16, torch.float32),    # ragged last segment
    (2, 4, 2, 64, 32, 16, torch.float32),    # GQA 2, batch 2
    (1, 2, 2, 8, 32, 1, torch.float32),      # one-token segments
    (1, 4, 2, 100, 64, 32, torch.bfloat16),  # ragged, GQA 2
    (1, 2, 1, 150, 128, 64, torch.bfloat16),  # d = 128, ragged
    (1, 1, 1, 300, 64, 300, torch.bfloat16),  # one segment
    (1, 8, 2, 300, 128, 130, torch.bfloat16),  # GQA 4 (four query heads per block), ragged
    (1, 4, 1, 5, 128, 1, torch.bfloat16),    # d = 128, one-token segments
    (1, 2, 1, 6, 64, 1, torch.bfloat16),     # d = 64, one-token segments
    (1, 2, 2, 7, 32, 1, torch.bfloat16),     # d = 32 (row kernels), one-token segments
    (2, 4, 1, 45, 128, 20, torch.bfloat16),  # d = 128, segments shorter than a 32-token chunk
]
IDS = [f"B{c[0]}Hq{c[1]}Hkv{c[2]}L{c[3]}d{c[4]}N{c[5]}{str(c[6])[6:]}" for c in CASES]


def run_case(lib, case, rule, seed, with_final=True, dv=None, m0_scale=0.3):
    B, Hq, Hkv, L, d, N, dt = case
    dv = d if dv is None else dv
    inp = random_inputs(B, Hq, Hkv, L, d, dt, DEV, seed=seed, m0_scale=m0_scale, dv=dv)
    g = torch.Generator(device="cpu").manual_seed(seed + 1)
    d_out = torch.randn(B, Hq, L, dv, generator=g).to(dt).to(DEV)
    dM_f = torch.randn(B, Hkv, d, dv, generator=g).to(DEV) if with_final else None
    dz_f = torch.randn(B, Hkv, d, generator=g).to(DEV) if with_final else None
    out, _, _, lse = lib.forward_train(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"],
                                       inp["z0"], N, rule)
    grads = lib.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"], N, rule,
                         out, lse, d_out, dM_f, dz_f)
    torch.cuda.synchronize()
    f64 = {k: synth.to_f64(v) for k, v in inp.items()}
    ref = oracle.backward(f64["q"], f64["k"], f64["v"], f64["beta"], f64["M0"], f64["z0"], N, rule,
                          synth.to_f64(d_out),
                          None if dM_f is None else synth.to_f64(dM_f),
                          None if dz_f is None else synth.to_f64(dz_f))
    names = ("dq", "dk", "dv", "dbeta", "dM0", "dz0")
    errs = {}
    for name, x, r in zip(names, grads, ref):
        x = synth.to_f64(x)
        if name == "dbeta":
            errs[name] = np.abs(x - r).max() / max(np.abs(r).max(), 1e-30)
        else:
            errs[name] = oracle.slice_errors(x, r)
    return errs, (inp, lse)


@pytest.mark.parametrize("case", CASES, ids=IDS)
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_gradients_match_the_oracle(lib, case, rule):
    _say(f"{case} {rule}")
    errs, _ = run_case(lib, case, rule, seed=case[3] + case[5])
    _say("errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    tol = TOL[case[6]]
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (bad, tol)


KV_PAIRS = [(32, 64), (32, 128), (64, 32), (64, 128), (128, 32), (128, 64)]


@pytest.mark.parametrize("pair", KV_PAIRS, ids=[f"dk{a}dv{b}" for a, b in KV_PAIRS])
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_gradients_with_kv_widths_match_the_oracle(lib, pair, dt, rule):
    """infini_attn_backward_kv (after infini_attn_forward_train_kv): every
    gradient against the oracle, for every ordered pair of widths, with GQA,
    a ragged last segment and final-state gradients."""
    dk, dv = pair
    case = (1, 4, 2, 70, dk, 32, dt)
    _say(f"kv widths {case} d_value {dv} {rule}")
    errs, _ = run_case(lib, case, rule, seed=dk + 7 * dv, dv=dv)
    _say("errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    tol = TOL[dt]
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (bad, tol)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_without_final_state_gradients(lib, dt):
    case = (1, 2, 1, 48, 64, 16, dt)
    _say(f"no dM_final / dz_final {case}")
    errs, _ = run_case(lib, case, "delta", seed=5, with_final=False)
    _say("errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL[dt], errs


@pytest.mark.parametrize("d", [64, 128])
def test_small_initial_z(lib, d):
    """M0 = 0 and z0 = 1e-6: the delta rule's transition I + A_s, A_s =
    -Phi^T diag(1/den) Phi with den = Phi z_{s-1}, has entries of order 1e6 in
    the first segment, so the state gradient's reversed chain is as sensitive
    to how A_s is formed as it gets (bf16, GQA 4, four segments, ragged).

    dM0 takes a bound of its own, 1e-3: with A_s formed from float operands
    (d = 64) or from bf16 hi/lo pairs (d = 128) it comes out near 3.4e-4; A_s
    from one bf16 product per term puts it near 3e-3."""
    case = (1, 4, 1, 200, d, 56, torch.bfloat16)
    _say(f"small z0 {case}")
    errs, _ = run_case(lib, case, "delta", seed=3 * d, m0_scale=0.0)
    _say("errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL[torch.bfloat16], errs
    assert errs["dM0"] <= 1e-3, errs


def test_llama_head_shape_two_segments(lib):
    """d = 128, 4 query heads on one KV head, two 2048-token segments, bf16,
    delta rule: the Llama-3-8B head shape at two segments."""
    case = (1, 4, 1, 4096, 128, 2048, torch.bfloat16)
    _say(f"llama head shape {case}")
    errs, _ = run_case(lib, case, "delta", seed=11)
    _say("errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL[torch.bfloat16], errs


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d,N,L,Hq", [(32, 16, 40, 2), (128, 64, 150, 2), (64, 256, 300, 2),
                                      (128, 320, 700, 4)])
def test_lse_is_the_log2_sum_exp_of_the_scaled_scores(lib, dt, d, N, L, Hq):
    _say(f"lse d{d} N{N} L{L} Hq{Hq} {dt}")
    B, Hkv = 1, 1
    inp = random_inputs(B, Hq, Hkv, L, d, dt, DEV, seed=d + N, m0_scale=0.3)
    _, _, _, lse = lib.forward_train(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"],
                                     inp["z0"], N, "linear")
    torch.cuda.synchronize()
    q, k = synth.to_f64(inp["q"]), synth.to_f64(inp["k"])
    c = 1.0 / math.sqrt(d)
    ref = np.empty((B, Hq, L))
    for h in range(Hq):
        for s0 in range(0, L, N):
            s1 = min(s0 + N, L)
            sc = (q[0, h, s0:s1] @ k[0, 0, s0:s1].T) * c
            sc = np.where(np.triu(np.ones((s1 - s0,) * 2, bool), 1), -np.inf, sc)
            m = sc.max(axis=1, keepdims=True)
            ref[0, h, s0:s1] = (m[:, 0] + np.log(np.exp(sc - m).sum(axis=1))) / math.log(2)
    err = np.abs(synth.to_f64(lse) - ref).max()
    _say(f"lse max abs error {err:.2e}")
    # bf16: the row sums are of bf16-rounded probabilities (2^-9 relative)
    assert err <= (1e-5 if dt == torch.float32 else 1e-2)
