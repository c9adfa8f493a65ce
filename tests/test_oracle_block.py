"""Pins of the oracle's projections around the block (oracle/block.py).

Scaled permutation (and selection) weights make every projected value one
input feature times a constant, so the expected q, k, v and y follow from
index arithmetic alone, element by element, with no matrix product and no
reshape; the attention in between is the already pinned oracle forward.
Plausible mistakes in the head split or the concatenation, planted in the
oracle on the CPU, fail these checks. Everything runs in float64.
"""

import numpy as np
import pytest

import oracle
from oracle import block as blk

RULES = ["linear", "delta"]


def perm_weights(rng, Hq, Hkv, d, dv=None, scales=(0.5, 2.0, -1.5, 3.0)):
    """d_model = Hq max(d, dv); W_q and W_k / W_v scaled selections of
    distinct input features (W_q a permutation when d_model = Hq d), W_o a
    scaled selection of distinct gated features. Query and key heads are d
    wide, value heads dv wide."""
    dv = d if dv is None else dv
    dm = Hq * max(d, dv)
    a_q, a_k, a_v, a_o = scales
    perm_q = rng.permutation(dm)[: Hq * d]
    sel_k = rng.permutation(dm)[: Hkv * d]
    sel_v = rng.permutation(dm)[: Hkv * dv]
    perm_o = rng.permutation(Hq * dv)
    w = np.zeros(((Hq + Hkv) * d + Hkv * dv, dm))
    for r in range(Hq * d):
        w[r, perm_q[r]] = a_q
    for r in range(Hkv * d):
        w[Hq * d + r, sel_k[r]] = a_k
    for r in range(Hkv * dv):
        w[(Hq + Hkv) * d + r, sel_v[r]] = a_v
    # output feature i reads gated feature perm_o[i] for i < Hq dv, nothing after
    w_o = np.zeros((dm, Hq * dv))
    for i in range(min(dm, Hq * dv)):
        w_o[i, perm_o[i]] = a_o
    return w, w_o, (perm_q, sel_k, sel_v, perm_o)


def expected_by_index(x, beta, M0, z0, N, rule, Hq, Hkv, d, idx, dv=None,
                      scales=(0.5, 2.0, -1.5, 3.0)):
    dv = d if dv is None else dv
    perm_q, sel_k, sel_v, perm_o = idx
    a_q, a_k, a_v, a_o = scales
    B, L, dm = x.shape
    q = np.empty((B, Hq, L, d))
    k = np.empty((B, Hkv, L, d))
    v = np.empty((B, Hkv, L, dv))
    for b in range(B):
        for t in range(L):
            for h in range(Hq):
                for j in range(d):
                    q[b, h, t, j] = a_q * x[b, t, perm_q[h * d + j]]
            for h in range(Hkv):
                for j in range(d):
                    k[b, h, t, j] = a_k * x[b, t, sel_k[h * d + j]]
                for j in range(dv):
                    v[b, h, t, j] = a_v * x[b, t, sel_v[h * dv + j]]
    out, M, z = oracle.forward(q, k, v, beta, M0, z0, N, rule)
    y = np.zeros((B, L, dm))
    for b in range(B):
        for t in range(L):
            for i in range(min(dm, Hq * dv)):
                f = perm_o[i]
                y[b, t, i] = a_o * out[b, f // dv, t, f % dv]
    return y, M, z


def make(rng, B, L, Hq, Hkv, d, m0=0.3, dv=None):
    dv = d if dv is None else dv
    x = rng.standard_normal((B, L, Hq * max(d, dv)))
    beta = rng.standard_normal(Hq)
    M0 = m0 * rng.standard_normal((B, Hkv, d, dv))
    z0 = 0.5 + rng.random((B, Hkv, d))
    return x, beta, M0, z0


# B, L, Hq, Hkv, d (key width), seg_len, value width
CASES = [(1, 7, 2, 1, 3, 3, 3), (2, 6, 4, 2, 2, 4, 2), (2, 7, 4, 2, 2, 3, 3),
         (1, 8, 2, 2, 4, 3, 2)]


def check_perm(rule, case, seed=0):
    B, L, Hq, Hkv, d, N, dv = case
    rng = np.random.default_rng(seed)
    x, beta, M0, z0 = make(rng, B, L, Hq, Hkv, d, dv=dv)
    w, w_o, idx = perm_weights(rng, Hq, Hkv, d, dv)
    y, M, z = blk.block_forward(x, w, w_o, beta, M0, z0, N, rule, Hq, Hkv, d, dv)
    ye, Me, ze = expected_by_index(x, beta, M0, z0, N, rule, Hq, Hkv, d, idx, dv)
    return max(np.abs(y - ye).max(), np.abs(M - Me).max(), np.abs(z - ze).max())


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("case", CASES, ids=["B1L7Hq2Hkv1", "B2L6Hq4Hkv2", "dk2dv3", "dk4dv2"])
def test_permutation_weights_match_index_arithmetic(rule, case):
    assert check_perm(rule, case) < 1e-12


@pytest.mark.parametrize("rule", RULES)
def test_y_is_linear_in_the_output_weight(rule):
    rng = np.random.default_rng(1)
    B, L, Hq, Hkv, d, N, dm = 2, 9, 4, 2, 3, 4, 10
    x = rng.standard_normal((B, L, dm))
    w = rng.standard_normal(((Hq + 2 * Hkv) * d, dm)) / np.sqrt(dm)
    w1, w2 = rng.standard_normal((2, dm, Hq * d))
    beta = rng.standard_normal(Hq)
    M0 = 0.3 * rng.standard_normal((B, Hkv, d, d))
    z0 = 0.5 + rng.random((B, Hkv, d))
    y1, M1, z1 = blk.block_forward(x, w, w1, beta, M0, z0, N, rule, Hq, Hkv, d)
    y2, M2, z2 = blk.block_forward(x, w, w2, beta, M0, z0, N, rule, Hq, Hkv, d)
    y3, M3, z3 = blk.block_forward(x, w, w1 + w2, beta, M0, z0, N, rule, Hq, Hkv, d)
    np.testing.assert_allclose(y3, y1 + y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(M1, M3)
    np.testing.assert_array_equal(z1, z2)


@pytest.mark.parametrize("rule", RULES)
def test_outputs_are_homogeneous_in_the_value_weights(rule):
    # from M0 = 0, both rules give M and A linear in V: scaling the value rows
    # of the input weight by c scales y and M by c and leaves z alone
    rng = np.random.default_rng(2)
    B, L, Hq, Hkv, d, N, dm = 1, 10, 4, 2, 3, 4, 8
    x = rng.standard_normal((B, L, dm))
    w = rng.standard_normal(((Hq + 2 * Hkv) * d, dm)) / np.sqrt(dm)
    w_o = rng.standard_normal((dm, Hq * d))
    beta = rng.standard_normal(Hq)
    M0 = np.zeros((B, Hkv, d, d))
    z0 = 0.5 + rng.random((B, Hkv, d))
    c = -2.5
    wc = w.copy()
    wc[(Hq + Hkv) * d:] *= c
    y, M, z = blk.block_forward(x, w, w_o, beta, M0, z0, N, rule, Hq, Hkv, d)
    yc, Mc, zc = blk.block_forward(x, wc, w_o, beta, M0, z0, N, rule, Hq, Hkv, d)
    np.testing.assert_allclose(yc, c * y, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Mc, c * M, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(zc, z, rtol=1e-14)


# ---- planted mistakes: each must fail the permutation check ----------------

def _kv_swapped(x, w_qkv, Hq, Hkv, d, dv=None, _f=blk.project_qkv):
    q, k, v = _f(x, w_qkv, Hq, Hkv, d, dv)
    return q, v, k


def _value_heads_key_wide(x, w_qkv, Hq, Hkv, d, dv=None):
    # value heads cut at the key width: the plausible slip with two widths
    B, L, _ = x.shape
    y = np.asarray(x) @ np.asarray(w_qkv).T
    heads = lambda cols, H, wd: y[..., cols].reshape(B, L, H, wd).transpose(0, 2, 1, 3)
    q = heads(slice(0, Hq * d), Hq, d)
    k = heads(slice(Hq * d, (Hq + Hkv) * d), Hkv, d)
    n = y.shape[-1] - (Hq + Hkv) * d
    v = y[..., (Hq + Hkv) * d:].reshape(B, L, n // Hkv, Hkv).transpose(0, 3, 1, 2)
    return q, k, v


def _split_without_transpose(x, w_qkv, Hq, Hkv, d, dv=None):
    B, L, _ = x.shape
    y = np.asarray(x) @ np.asarray(w_qkv).T
    q = y[..., : Hq * d].reshape(B, Hq, L, d)
    k = y[..., Hq * d:(Hq + Hkv) * d].reshape(B, Hkv, L, d)
    v = y[..., (Hq + Hkv) * d:].reshape(B, Hkv, L, d)
    return q, k, v


def _out_weight_not_transposed(a, w_o):
    B, Hq, L, d = a.shape
    return a.transpose(0, 2, 1, 3).reshape(B, L, Hq * d) @ w_o


def _concat_feature_major(a, w_o):
    B, Hq, L, d = a.shape
    return a.transpose(0, 2, 3, 1).reshape(B, L, Hq * d) @ w_o.T


MUTANTS = {
    "key and value slices swapped": ("project_qkv", _kv_swapped),
    "head split without the transpose": ("project_qkv", _split_without_transpose),
    "output weight not transposed": ("project_out", _out_weight_not_transposed),
    "heads concatenated feature-major": ("project_out", _concat_feature_major),
    "value heads split at the wrong width": ("project_qkv", _value_heads_key_wide),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_fails_the_permutation_check(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(blk, attr, fn)
    case = CASES[2] if name == "value heads split at the wrong width" else CASES[1]
    assert check_perm("delta", case) > 1e-3, name
