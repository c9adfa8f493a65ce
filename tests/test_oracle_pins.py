"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these recompute the oracle's own formula the oracle's way: each check
is a library routine, a closed form in a different association order, a
hand-worked example, or an invariant, chosen so that a dropped term, a wrong
sign, a wrong index or a transposed operand in the oracle fails at least one.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import (feature_map, forward, gate_weight, local_causal_attention,
                    memory_retrieval, memory_update)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BIG = 40.0  # sigmoid(40) rounds to exactly 1.0 in float64, sigmoid(-40) to ~4e-18


def case(rng, B=1, Hq=2, Hkv=2, L=12, d=4, dv=None, m0_scale=0.0, z0=None):
    dv = d if dv is None else dv
    q = rng.standard_normal((B, Hq, L, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, dv))
    beta = rng.standard_normal(Hq)
    M0 = m0_scale * rng.standard_normal((B, Hkv, d, dv))
    if z0 is None:
        z0 = rng.uniform(0.5, 2.0, (B, Hkv, d))
    else:
        z0 = np.full((B, Hkv, d), z0)
    return q, k, v, beta, M0, z0


def sig_scalar(x):
    return x + 1.0 if x > 0 else math.exp(x)


def outer_sum(phi, v):
    """sum_t phi_t (outer) v_t, with explicit per-token outer products."""
    acc = np.zeros((phi.shape[1], v.shape[1]))
    for t in range(phi.shape[0]):
        for i in range(phi.shape[1]):
            for j in range(v.shape[1]):
                acc[i, j] += phi[t, i] * v[t, j]
    return acc


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# --- sigma and the gate ------------------------------------------------------

def test_feature_map_is_elu_plus_one():
    x = np.concatenate([np.linspace(-30, 30, 601), np.random.default_rng(0).standard_normal(1000)])
    ref = torch.nn.functional.elu(torch.tensor(x, dtype=torch.float64), alpha=1.0) + 1.0
    # torch forms ELU as expm1(x) + 1, which is exact only to ~1e-16 absolute
    np.testing.assert_allclose(feature_map(x), ref.numpy(), rtol=1e-15, atol=1e-16)
    assert feature_map(0.0) == 1.0 and feature_map(1.0) == 2.0
    assert feature_map(-np.inf) == 0.0
    assert np.all(feature_map(x) > 0)


def test_gate_weight_is_logistic():
    for beta in (-BIG, -3.0, -0.25, 0.0, 0.5, 3.0, BIG):
        assert gate_weight(beta) == pytest.approx(scipy.special.expit(beta), rel=1e-15)
    assert gate_weight(BIG) == 1.0
    assert 0.0 < gate_weight(-BIG) < 1e-17
    assert gate_weight(0.0) == 0.5


# --- local causal attention ----------------------------------------------------

@pytest.mark.parametrize("n,d", [(1, 3), (5, 4), (17, 8)])
def test_local_attention_matches_sdpa(rng, n, d):
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    got = local_causal_attention(q, k, v)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None], torch.tensor(k)[None], torch.tensor(v)[None],
        is_causal=True)[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    # the same with a scalar softmax per row
    for t in range(n):
        s = [sum(q[t, i] * k[u, i] for i in range(d)) / math.sqrt(d) for u in range(t + 1)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        row = [sum(w[u] * v[u, j] for u in range(t + 1)) / sum(w) for j in range(d)]
        np.testing.assert_allclose(got[t], row, rtol=1e-12, atol=1e-13)


def test_local_attention_first_row_is_first_value(rng):
    q, k, v = (rng.standard_normal((6, 5)) for _ in range(3))
    np.testing.assert_array_equal(local_causal_attention(q, k, v)[0], v[0])


# --- the hand-worked example ---------------------------------------------------

def _worked():
    with open(os.path.join(GOLDEN, "worked_example_d2.json")) as f:
        g = json.load(f)
    inp = g["inputs"]
    q = np.array(inp["q"], float)[None, None]
    k = np.array(inp["k"], float)[None, None]
    v = np.array(inp["v"], float)[None, None]
    M0 = np.array(inp["M0"], float)[None, None]
    z0 = np.array(inp["z0"], float)[None, None]
    return g, q, k, v, M0, z0, inp["seg_len"]


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_worked_example(rule):
    g, q, k, v, M0, z0, N = _worked()
    exp = g["expected"]
    out_mem, M, z = forward(q, k, v, np.array([BIG]), M0, z0, N, rule)
    np.testing.assert_allclose(out_mem[0, 0], np.array(exp["a_mem"]), rtol=1e-15, atol=0)
    np.testing.assert_array_equal(M[0, 0], np.array(exp["M_final"][rule]))
    np.testing.assert_array_equal(z[0, 0], np.array(exp["z_final"]))
    out_dot, _, _ = forward(q, k, v, np.array([-BIG]), M0, z0, N, rule)
    for row, val in exp["a_dot_exact_rows"].items():
        np.testing.assert_allclose(out_dot[0, 0, int(row)], val, rtol=0, atol=1e-15)
    a = 1.0 / math.sqrt(2.0)
    np.testing.assert_allclose(out_dot[0, 0, 3], [1.0 + 1.0 / (1.0 + math.exp(-a)), 1.0],
                               rtol=1e-15, atol=1e-15)


# --- reductions to textbook computations --------------------------------------

@pytest.mark.parametrize("seg_len", [9, 64])
def test_single_segment_is_gated_causal_attention(rng, seg_len):
    """S = 1 and M0 = 0: out = (1 - g) causal SDPA, M = sum sigma(k) v^T under
    both rules, z = z0 + sum sigma(k)."""
    q, k, v, beta, M0, z0 = case(rng, B=2, Hq=4, Hkv=2, L=9, d=4)
    for rule in ("linear", "delta"):
        out, M, z = forward(q, k, v, beta, M0, z0, seg_len, rule)
        kr = torch.tensor(k).repeat_interleave(2, dim=1)
        vr = torch.tensor(v).repeat_interleave(2, dim=1)
        sdpa = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q), kr, vr, is_causal=True).numpy()
        g = scipy.special.expit(beta)[None, :, None, None]
        np.testing.assert_allclose(out, (1 - g) * sdpa, rtol=1e-12, atol=1e-13)
        for b in range(2):
            for j in range(2):
                phi = np.array([[sig_scalar(x) for x in row] for row in k[b, j]])
                np.testing.assert_allclose(M[b, j], outer_sum(phi, v[b, j]), rtol=1e-13)
                np.testing.assert_allclose(z[b, j], z0[b, j] + phi.sum(0), rtol=1e-15)


def test_linear_state_is_segmentation_independent(rng):
    q, k, v, beta, M0, z0 = case(rng, B=1, Hq=2, Hkv=1, L=13, d=3, dv=5, m0_scale=1.0)
    phi = feature_map(k[0, 0])
    M_ref = M0[0, 0] + outer_sum(phi, v[0, 0])
    z_ref = z0[0, 0] + phi.sum(0)
    for seg_len in (1, 2, 3, 5, 13, 20):
        _, M, z = forward(q, k, v, beta, M0, z0, seg_len, "linear")
        assert rel(M[0, 0], M_ref) < 1e-13
        assert rel(z[0, 0], z_ref) < 1e-15


@pytest.mark.parametrize("seg_len", [3, 4])
def test_retrieval_closed_form(rng, seg_len):
    """Linear rule, gate at 1: for a token t of segment s,
    A_mem_t = (sigma(q_t)M0 + sum_{u < sN} (sigma(q_t).sigma(k_u)) v_u)
              / (sigma(q_t).z0 + sum_{u < sN} sigma(q_t).sigma(k_u)),
    a block-strictly-causal quadratic form, evaluated token by token."""
    L, d = 11, 3
    q, k, v, _, M0, z0 = case(rng, B=1, Hq=1, Hkv=1, L=L, d=d, m0_scale=0.5)
    out, _, _ = forward(q, k, v, np.array([BIG]), M0, z0, seg_len, "linear")
    for t in range(L):
        s0 = (t // seg_len) * seg_len
        sq = [sig_scalar(x) for x in q[0, 0, t]]
        num = [sum(sq[i] * M0[0, 0, i, j] for i in range(d)) for j in range(d)]
        den = sum(sq[i] * z0[0, 0, i] for i in range(d))
        for u in range(s0):
            w = sum(sq[i] * sig_scalar(k[0, 0, u, i]) for i in range(d))
            den += w
            for j in range(d):
                num[j] += w * v[0, 0, u, j]
        np.testing.assert_allclose(out[0, 0, t], np.array(num) / den, rtol=1e-12)


def test_seg_len_one_is_causal_linear_attention(rng):
    """seg_len = 1: the memory path is linear attention over strictly earlier
    tokens, and the local path sees only the token itself."""
    L, d = 8, 4
    q, k, v, _, M0, z0 = case(rng, B=1, Hq=1, Hkv=1, L=L, d=d, z0=1e-6)
    out_mem, _, _ = forward(q, k, v, np.array([BIG]), M0, z0, 1, "linear")
    sq, sk = feature_map(q[0, 0]), feature_map(k[0, 0])
    for t in range(L):
        w = np.array([sq[t] @ sk[u] for u in range(t)])
        num = sum((w[u] * v[0, 0, u] for u in range(t)), np.zeros(d))
        den = sq[t] @ z0[0, 0] + w.sum()
        np.testing.assert_allclose(out_mem[0, 0, t], num / den, rtol=1e-12, atol=1e-300)
    out_dot, _, _ = forward(q, k, v, np.array([-BIG]), M0, z0, 1, "linear")
    np.testing.assert_allclose(out_dot[0, 0], v[0, 0], rtol=1e-15, atol=1e-15)


# --- the delta rule -------------------------------------------------------------

def test_delta_zero_residual_keeps_memory(rng):
    """Values equal to what the memory already predicts leave M unchanged,
    while z still grows."""
    d, n = 4, 6
    q, k, v, beta, M0, z0 = case(rng, B=1, Hq=1, Hkv=1, L=2 * n, d=d)
    # after a first segment of random values, make the second segment's values
    # equal to the retrieval through its own keys
    _, M1, z1 = forward(q[:, :, :n], k[:, :, :n], v[:, :, :n], beta, M0, z0, n, "delta")
    v2 = v.copy()
    for t in range(n, 2 * n):
        phi = np.array([sig_scalar(x) for x in k[0, 0, t]])
        v2[0, 0, t] = (phi @ M1[0, 0]) / (phi @ z1[0, 0])
    _, M2, z2 = forward(q, k, v2, beta, M0, z0, n, "delta")
    np.testing.assert_allclose(M2[0, 0], M1[0, 0], rtol=0, atol=1e-12 * np.abs(M1).max())
    np.testing.assert_allclose(z2[0, 0], z1[0, 0] + feature_map(k[0, 0, n:]).sum(0), rtol=1e-15)
    # the linear rule is not invariant to the same values
    _, M2_lin, _ = forward(q, k, v2, beta, M0, z0, n, "linear")
    assert rel(M2_lin[0, 0], M1[0, 0]) > 1e-3


def test_delta_equals_linear_from_zero_memory(rng):
    q, k, v, beta, M0, z0 = case(rng, B=1, Hq=2, Hkv=2, L=10, d=4)
    a = forward(q, k, v, beta, M0, z0, 10, "delta")
    b = forward(q, k, v, beta, M0, z0, 10, "linear")
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    a = forward(q, k, v, beta, M0, z0, 5, "delta")
    b = forward(q, k, v, beta, M0, z0, 5, "linear")
    assert rel(a[1], b[1]) > 1e-3  # the second segment sees a nonzero memory


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_scalar_memory_closed_form(rng, rule):
    """d = 1: A_mem = M/z whatever the query; the delta rule reduces to
    M_s = M_{s-1} (1 - sum_t phi_t / z_{s-1}) + sum_t phi_t v_t."""
    L, N = 10, 3
    q, k, v, _, M0, z0 = case(rng, B=1, Hq=1, Hkv=1, L=L, d=1, m0_scale=1.0)
    out, M, z = forward(q, k, v, np.array([BIG]), M0, z0, N, rule)
    Ms, zs = M0[0, 0, 0, 0], z0[0, 0, 0]
    for s0 in range(0, L, N):
        t1 = min(s0 + N, L)
        np.testing.assert_allclose(out[0, 0, s0:t1, 0], Ms / zs, rtol=1e-13)
        phi = [sig_scalar(k[0, 0, t, 0]) for t in range(s0, t1)]
        pv = sum(p * v[0, 0, t, 0] for p, t in zip(phi, range(s0, t1)))
        if rule == "delta":
            Ms = Ms * (1.0 - sum(phi) / zs) + pv
        else:
            Ms = Ms + pv
        zs = zs + sum(phi)
    assert M[0, 0, 0, 0] == pytest.approx(Ms, rel=1e-12)
    assert z[0, 0, 0] == pytest.approx(zs, rel=1e-15)


def test_delta_affine_transition_form(rng):
    """The delta rule is affine in M with a transition that depends on K and z
    only: M_s = (I - Phi^T diag(1/(Phi z_{s-1})) Phi) M_{s-1} + Phi^T V."""
    L, N, d, dv = 12, 4, 3, 5
    q, k, v, beta, M0, z0 = case(rng, B=1, Hq=1, Hkv=1, L=L, d=d, dv=dv, m0_scale=1.0)
    _, M, z = forward(q, k, v, beta, M0, z0, N, "delta")
    Ms, zs = M0[0, 0].copy(), z0[0, 0].copy()
    for s0 in range(0, L, N):
        Phi = feature_map(k[0, 0, s0:s0 + N])
        A = np.eye(d) - Phi.T @ np.diag(1.0 / (Phi @ zs)) @ Phi
        Ms = A @ Ms + Phi.T @ v[0, 0, s0:s0 + N]
        zs = zs + Phi.sum(0)
    assert rel(M[0, 0], Ms) < 1e-12
    assert rel(z[0, 0], zs) < 1e-15


# --- the gate and the whole forward ---------------------------------------------

@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_gate_mixes_the_two_paths(rng, rule):
    q, k, v, beta, M0, z0 = case(rng, B=1, Hq=3, Hkv=1, L=10, d=4, m0_scale=0.3)
    mem, _, _ = forward(q, k, v, np.full(3, BIG), M0, z0, 4, rule)
    dot, _, _ = forward(q, k, v, np.full(3, -BIG), M0, z0, 4, rule)
    out, _, _ = forward(q, k, v, beta, M0, z0, 4, rule)
    g = scipy.special.expit(beta)[None, :, None, None]
    np.testing.assert_allclose(out, g * mem + (1 - g) * dot, rtol=1e-12, atol=1e-14)
    half, _, _ = forward(q, k, v, np.zeros(3), M0, z0, 4, rule)
    np.testing.assert_allclose(half, 0.5 * (mem + dot), rtol=1e-12, atol=1e-14)


def test_constant_values_give_constant_output(rng):
    """Linear rule, V = c on every row and M0 = z0 c^T: both attentions average
    a constant, so out = c everywhere and M_s = z_s c^T."""
    B, Hq, Hkv, L, d = 1, 2, 1, 11, 4
    q, k, _, beta, _, z0 = case(rng, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d)
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (B, Hkv, L, d)).copy()
    M0 = z0[..., :, None] * c[None, None, None, :]
    out, M, z = forward(q, k, v, beta, M0, z0, 3, "linear")
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=1e-12)
    np.testing.assert_allclose(M[0, 0], np.outer(z[0, 0], c), rtol=1e-12)


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_joint_linearity_in_values_and_memory(rng, rule):
    q, k, v1, beta, M1, z0 = case(rng, B=1, Hq=2, Hkv=1, L=10, d=3, m0_scale=1.0)
    v2 = rng.standard_normal(v1.shape)
    M2 = rng.standard_normal(M1.shape)
    a = forward(q, k, v1, beta, M1, z0, 4, rule)
    b = forward(q, k, v2, beta, M2, z0, 4, rule)
    c = forward(q, k, 2.0 * v1 - 3.0 * v2, beta, 2.0 * M1 - 3.0 * M2, z0, 4, rule)
    for x, y, w in zip(a[:2], b[:2], c[:2]):
        np.testing.assert_allclose(w, 2.0 * x - 3.0 * y, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(c[2], a[2])


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_gqa_equals_mha_on_repeated_kv(rng, rule):
    G = 3
    q, k, v, beta, M0, z0 = case(rng, B=2, Hq=6, Hkv=2, L=9, d=4, m0_scale=0.5)
    out, M, z = forward(q, k, v, beta, M0, z0, 4, rule)
    rep = lambda a: np.repeat(a, G, axis=1)
    out2, M2, z2 = forward(q, rep(k), rep(v), beta, rep(M0), rep(z0), 4, rule)
    np.testing.assert_allclose(out, out2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(rep(M), M2, rtol=1e-13)
    np.testing.assert_allclose(rep(z), z2, rtol=1e-15)


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_batch_and_head_permutation(rng, rule):
    q, k, v, beta, M0, z0 = case(rng, B=3, Hq=4, Hkv=4, L=7, d=3, m0_scale=0.5)
    out, M, z = forward(q, k, v, beta, M0, z0, 3, rule)
    pb, ph = np.array([2, 0, 1]), np.array([3, 1, 0, 2])
    P = lambda a: a[pb][:, ph]
    out2, M2, z2 = forward(P(q), P(k), P(v), beta[ph], P(M0), P(z0), 3, rule)
    np.testing.assert_allclose(out2, P(out), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(M2, P(M), rtol=1e-14)
    np.testing.assert_allclose(z2, P(z), rtol=1e-15)


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_chunked_calls_carry_the_state(rng, rule):
    q, k, v, beta, M0, z0 = case(rng, B=1, Hq=2, Hkv=2, L=14, d=4)
    out, M, z = forward(q, k, v, beta, M0, z0, 4, rule)
    cut = 8
    o1, M1, z1 = forward(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], beta, M0, z0, 4, rule)
    o2, M2, z2 = forward(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], beta, M1, z1, 4, rule)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(M2, M, rtol=1e-13)
    np.testing.assert_allclose(z2, z, rtol=1e-15)


def test_normaliser_is_monotone_and_positive(rng):
    q, k, v, beta, M0, z0 = case(rng, B=1, Hq=1, Hkv=1, L=12, d=5, z0=1e-6)
    prev = z0[0, 0]
    for L in range(3, 13, 3):
        _, _, z = forward(q[:, :, :L], k[:, :, :L], v[:, :, :L], beta, M0, z0, 3, "delta")
        assert np.all(z[0, 0] > prev)
        prev = z[0, 0]


def test_sampling_options_match_full_run(rng):
    q, k, v, beta, M0, z0 = case(rng, B=2, Hq=4, Hkv=2, L=12, d=3)
    out, M, z = forward(q, k, v, beta, M0, z0, 4, "delta")
    out_s, M_s, z_s = forward(q, k, v, beta, M0, z0, 4, "delta",
                              units=[(1, 0)], out_segments={0, 2})
    np.testing.assert_array_equal(M_s[1, 0], M[1, 0])
    np.testing.assert_array_equal(z_s[1, 0], z[1, 0])
    assert np.isnan(M_s[0]).all() and np.isnan(out_s[0]).all()
    for s in (0, 2):
        np.testing.assert_array_equal(out_s[1, 0:2, 4 * s:4 * s + 4], out[1, 0:2, 4 * s:4 * s + 4])
    assert np.isnan(out_s[1, :, 4:8]).all()


def test_unknown_rule_is_rejected(rng):
    q, k, v, beta, M0, z0 = case(rng)
    with pytest.raises(ValueError):
        forward(q, k, v, beta, M0, z0, 4, "hebbian")


def test_compare_metric():
    ref = np.array([[1.0, -2.0], [0.5, 4.0]])
    x = ref + np.array([[0.0, 0.04], [0.0, 0.0]])
    assert oracle.max_rel_err(x, ref) == pytest.approx(0.01)
    assert oracle.max_rel_err(x, ref, elementwise=True) == pytest.approx(0.02)
    assert oracle.max_rel_err(np.array([np.inf]), np.array([1.0])) == float("inf")
