"""Pins of the row-restricted oracle (oracle.forward_rows, used where a
segment is too long for its N x N score matrix): on small streams it equals
the full oracle forward row for row, and attend_last_row equals the last row
of the full causal attention of the same block. A planted mistake (the
diagonal left out of the prefix) fails. float64, CPU."""

import numpy as np
import pytest

import oracle
from oracle import infini_attention as ia


def make(B, Hq, Hkv, L, d, seed):
    r = np.random.default_rng(seed)
    return dict(q=r.standard_normal((B, Hq, L, d)), k=r.standard_normal((B, Hkv, L, d)),
                v=r.standard_normal((B, Hkv, L, d)), beta=r.standard_normal(Hq),
                M0=0.3 * r.standard_normal((B, Hkv, d, d)), z0=0.5 + r.random((B, Hkv, d)))


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("shape", [(1, 2, 1, 23, 4, 7), (2, 4, 2, 16, 3, 16), (1, 1, 1, 9, 2, 1)],
                         ids=["ragged-gqa2", "one-segment-gqa2", "one-token-segments"])
def test_rows_equal_the_full_forward(rule, shape):
    B, Hq, Hkv, L, d, N = shape
    x = make(B, Hq, Hkv, L, d, seed=L + N)
    out, M, z = oracle.forward(x["q"], x["k"], x["v"], x["beta"], x["M0"], x["z0"], N, rule)
    rows = list(range(L))[::-1]  # every row, in an order of its own
    got, Mr, zr = oracle.forward_rows(x["q"], x["k"], x["v"], x["beta"], x["M0"], x["z0"], N,
                                      rule, rows)
    np.testing.assert_allclose(got, out[:, :, rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Mr, M, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(zr, z, rtol=1e-12, atol=1e-12)


def test_attend_last_row_is_the_last_causal_row():
    r = np.random.default_rng(3)
    q, k, v = r.standard_normal((3, 11, 5))
    full = oracle.local_causal_attention(q, k, v)
    for t in range(11):
        np.testing.assert_allclose(oracle.attend_last_row(q[t], k[:t + 1], v[:t + 1]),
                                   oracle.local_causal_attention(q[:t + 1], k[:t + 1],
                                                                 v[:t + 1])[-1],
                                   rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(oracle.attend_last_row(q[t], k[:t + 1], v[:t + 1]), full[t],
                                   rtol=1e-12, atol=1e-13)


def test_planted_mistake_diagonal_left_out_fails(monkeypatch):
    x = make(1, 1, 1, 12, 3, seed=1)
    out, _, _ = oracle.forward(x["q"], x["k"], x["v"], x["beta"], x["M0"], x["z0"], 6, "linear")
    real = ia.attend_last_row

    def without_diagonal(q_t, k_prefix, v_prefix):
        if len(k_prefix) == 1:
            return real(q_t, k_prefix, v_prefix)
        return real(q_t, k_prefix[:-1], v_prefix[:-1])

    monkeypatch.setattr(ia, "attend_last_row", without_diagonal)
    got, _, _ = ia.forward_rows(x["q"], x["k"], x["v"], x["beta"], x["M0"], x["z0"], 6, "linear",
                                range(12))
    assert np.abs(got - out).max() > 1e-3
