"""Pins of the oracle's backward pass (oracle/gradients.py).

The gradients are checked against central finite differences of the oracle
forward, a definition independent of the chain-rule derivation: for a scalar
loss  sum(d_out * out) + sum(dM_final * M_final) + sum(dz_final * z_final),
every element of every input is nudged by +-h and the loss difference is
compared with the returned gradient. Plausible mistakes planted in the
backward (a dropped term, a wrong carry, a wrong derivative) are shown to
fail the same check. Everything here runs on the CPU in float64.
"""

import numpy as np
import pytest

import oracle
from oracle import gradients as bw

CASES = [
    # B, Hq, Hkv, L, d (the key width), seg_len[, d_value]
    (1, 2, 1, 7, 3, 3),   # ragged last segment, two query heads on one KV head
    (2, 4, 2, 6, 2, 2),   # GQA 2, batch 2
    (1, 1, 1, 5, 3, 8),   # one segment (seg_len > L)
    (1, 1, 1, 4, 2, 1),   # one-token segments
    (1, 2, 1, 7, 2, 3, 3),  # values wider than keys, ragged
    (1, 2, 2, 6, 3, 4, 2),  # values narrower than keys
]


def make(case, seed):
    B, Hq, Hkv, L, d, N = case[:6]
    dv = case[6] if len(case) > 6 else d
    r = np.random.default_rng(seed)
    x = dict(
        q=r.standard_normal((B, Hq, L, d)),
        k=r.standard_normal((B, Hkv, L, d)),
        v=r.standard_normal((B, Hkv, L, dv)),
        beta=r.standard_normal(Hq),
        M0=0.3 * r.standard_normal((B, Hkv, d, dv)),
        z0=0.5 + r.random((B, Hkv, d)),
    )
    cot = dict(
        d_out=r.standard_normal((B, Hq, L, dv)),
        dM_final=r.standard_normal((B, Hkv, d, dv)),
        dz_final=r.standard_normal((B, Hkv, d)),
    )
    return x, cot, N


def loss(x, cot, N, rule):
    out, M, z = oracle.forward(x["q"], x["k"], x["v"], x["beta"], x["M0"], x["z0"], N, rule)
    return (cot["d_out"] * out).sum() + (cot["dM_final"] * M).sum() + (cot["dz_final"] * z).sum()


def fd_grads(x, cot, N, rule, h=1e-6):
    g = {}
    for name, arr in x.items():
        gr = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            up = loss(x, cot, N, rule)
            arr[idx] = keep - h
            dn = loss(x, cot, N, rule)
            arr[idx] = keep
            gr[idx] = (up - dn) / (2 * h)
        g[name] = gr
    return g


def analytic(x, cot, N, rule):
    dq, dk, dv, dbeta, dM0, dz0 = bw.backward(x["q"], x["k"], x["v"], x["beta"], x["M0"], x["z0"],
                                              N, rule, cot["d_out"], cot["dM_final"],
                                              cot["dz_final"])
    return dict(q=dq, k=dk, v=dv, beta=dbeta, M0=dM0, z0=dz0)


def worst_rel(a, b):
    return max(np.abs(a[n] - b[n]).max() / max(np.abs(b[n]).max(), 1e-12) for n in b)


_FD = {}


def fd_cached(case, rule, seed):
    key = (case, rule, seed)
    if key not in _FD:
        x, cot, N = make(case, seed)
        _FD[key] = (x, cot, N, fd_grads(x, cot, N, rule))
    return _FD[key]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}L{c[3]}d{c[4]}N{c[5]}"
                                             + (f"dv{c[6]}" if len(c) > 6 else "")
                                             for c in CASES])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_backward_matches_finite_differences(case, rule):
    x, cot, N, fd = fd_cached(case, rule, 7)
    an = analytic(x, cot, N, rule)
    for name in fd:
        err = np.abs(an[name] - fd[name]).max() / max(np.abs(fd[name]).max(), 1e-12)
        assert err < 1e-6, (name, err)


def test_without_cotangent_on_state_the_state_gradients_come_from_out_only():
    # dM_final = dz_final = 0: the last segment's update gets no gradient, so
    # its keys and values get gradients from the local path only
    x, cot, N = make((1, 1, 1, 6, 2, 3), 3)
    dq, dk, dv, dbeta, dM0, dz0 = bw.backward(x["q"], x["k"], x["v"], x["beta"], x["M0"],
                                              x["z0"], N, "delta", cot["d_out"])
    _, dk_a, dv_a = bw.local_attention_backward(
        x["q"][0, 0, 3:], x["k"][0, 0, 3:], x["v"][0, 0, 3:],
        (1 - oracle.gate_weight(x["beta"][0])) * cot["d_out"][0, 0, 3:])
    np.testing.assert_allclose(dk[0, 0, 3:], dk_a, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv[0, 0, 3:], dv_a, rtol=1e-12, atol=1e-14)


# ---- planted mistakes: each must fail the finite-difference check -----------

def _no_dz_carry(k_s, v_s, M_prev, z_prev, dM, dz, rule, _f=bw.update_backward):
    dk_s, dv_s, dM_prev, dz_prev = _f(k_s, v_s, M_prev, z_prev, dM, dz, rule)
    return dk_s, dv_s, dM_prev, dz_prev - dz  # z_s = z_prev + ... not carried


def _no_retrieval_dM(q_s, M_prev, z_prev, da_mem, _f=bw.retrieval_backward):
    dq, dM, dz = _f(q_s, M_prev, z_prev, da_mem)
    return dq, 0.0 * dM, dz


def _softmax_without_rowsum(q_s, k_s, v_s, da_dot):
    n, d = q_s.shape
    s = (q_s @ k_s.T) / np.sqrt(d)
    s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ds = p * (da_dot @ v_s.T)  # the row-sum term dropped
    return ds @ k_s / np.sqrt(d), ds.T @ q_s / np.sqrt(d), p.T @ da_dot


def _delta_without_dc(k_s, v_s, M_prev, z_prev, dM, dz, rule):
    phi = oracle.feature_map(k_s)
    dphi = np.broadcast_to(dz, phi.shape).copy()
    c = phi @ z_prev
    pred = (phi @ M_prev) / c[:, None]
    du = phi @ dM
    dphi += (v_s - pred) @ dM.T
    dp = -du / c[:, None]
    dphi += dp @ M_prev.T
    return dphi * bw.feature_map_grad(k_s), du, dM + phi.T @ dp, dz.copy()


MUTANTS = {
    "dz not carried through the update": ("update_backward", _no_dz_carry, "linear"),
    "retrieval gives M no gradient": ("retrieval_backward", _no_retrieval_dM, "linear"),
    "softmax backward without the row sum": ("local_attention_backward",
                                             _softmax_without_rowsum, "linear"),
    "sigma' = 1 everywhere": ("feature_map_grad", lambda x: np.ones_like(x), "delta"),
    "delta rule without the denominator term": ("update_backward", _delta_without_dc, "delta"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_fails_the_finite_difference_check(name, monkeypatch):
    attr, fn, rule = MUTANTS[name]
    case = (1, 2, 1, 7, 3, 3)
    x, cot, N, fd = fd_cached(case, rule, 7)
    monkeypatch.setattr(bw, attr, fn)
    an = analytic(x, cot, N, rule)
    assert worst_rel(an, fd) > 1e-3, name
