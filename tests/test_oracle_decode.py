"""Pins of the oracle's streaming decode step.

Token-by-token decoding of a stream must give what the segment-wise forward
gives on the whole stream: every output row, and the state at every segment
end ("Infini-Attention" (AI Wiki), "Why is the memory footprint bounded?":
the stream is processed segment by segment with only (M, z) carried). The
forward is pinned on its own (tests/test_oracle_pins.py), so a mistake in the
step's causal window, its GQA mapping, its retrieval or its fold of the
segment into the state fails here.
"""

import numpy as np
import pytest

import oracle


def stream(rng, B=2, Hq=4, Hkv=2, L=17, d=6, m0_scale=0.3):
    q = rng.standard_normal((B, Hq, L, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    beta = rng.standard_normal(Hq)
    M0 = m0_scale * rng.standard_normal((B, Hkv, d, d))
    z0 = rng.uniform(0.5, 2.0, (B, Hkv, d))
    return q, k, v, beta, M0, z0


def decode_all(q, k, v, beta, M0, z0, seg_len, rule):
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    M, z = M0.copy(), z0.copy()
    kc = np.zeros((B, Hkv, seg_len, d))
    vc = np.zeros((B, Hkv, seg_len, d))
    outs, states = [], {}
    for t in range(L):
        pos = t % seg_len
        o, M, z, kc, vc = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], beta, M, z, kc,
                                             vc, pos, seg_len, rule)
        outs.append(o)
        if pos == seg_len - 1:
            states[t + 1] = (M.copy(), z.copy())
    return np.stack(outs, axis=2), states


@pytest.mark.parametrize("rule", oracle.RULES)
@pytest.mark.parametrize("seg_len", [1, 5, 17, 40])
def test_decoding_a_stream_equals_the_forward(rng, rule, seg_len):
    q, k, v, beta, M0, z0 = stream(rng)
    out, states = decode_all(q, k, v, beta, M0, z0, seg_len, rule)
    ref, _, _ = oracle.forward(q, k, v, beta, M0, z0, seg_len, rule)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    for n, (M, z) in states.items():
        _, M_ref, z_ref = oracle.forward(q[:, :, :n], k[:, :, :n], v[:, :, :n], beta, M0, z0,
                                         seg_len, rule)
        np.testing.assert_allclose(M, M_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(z, z_ref, rtol=1e-12, atol=1e-12)


def test_first_token_of_a_segment_sees_only_itself(rng):
    """At pos 0 the softmax has one key: A_dot is the token's own value."""
    q, k, v, beta, M0, z0 = stream(rng, L=1)
    B, Hq, _, d = q.shape
    Hkv = k.shape[1]
    junk = rng.standard_normal((B, Hkv, 8, d))  # stale rows must not be read
    out, M, z, kc, _ = oracle.decode_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], beta, M0, z0, junk,
                                          junk, 0, 8, "delta")
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            j = h // G
            sq = oracle.feature_map(q[b, h, 0])
            a_mem = (sq @ M0[b, j]) / (sq @ z0[b, j])
            g = 1.0 / (1.0 + np.exp(-beta[h]))
            np.testing.assert_allclose(out[b, h], g * a_mem + (1 - g) * v[b, j, 0], rtol=1e-12)
    np.testing.assert_array_equal(M, M0)
    np.testing.assert_array_equal(z, z0)
    np.testing.assert_array_equal(kc[:, :, 0], k[:, :, 0])


def test_state_changes_only_at_the_segment_end(rng):
    q, k, v, beta, M0, z0 = stream(rng, L=4)
    B, Hq, L, d = q.shape
    kc = np.zeros((B, k.shape[1], 4, d))
    vc = np.zeros_like(kc)
    M, z = M0, z0
    for t in range(4):
        _, M1, z1, kc, vc = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], beta, M, z, kc,
                                               vc, t, 4, "linear")
        if t < 3:
            np.testing.assert_array_equal(M1, M0)
            np.testing.assert_array_equal(z1, z0)
        M, z = M1, z1
    assert not np.array_equal(M, M0)


def test_bad_position_is_rejected(rng):
    q, k, v, beta, M0, z0 = stream(rng, L=1)
    kc = np.zeros((2, 2, 4, 6))
    with pytest.raises(ValueError):
        oracle.decode_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], beta, M0, z0, kc, kc, 4, 4, "linear")


def _mutant(kind):
    """A plausible wrong decode step: the stream pin must reject it."""
    def step(q, k, v, beta, M, z, kc, vc, pos, seg_len, rule):
        M, z, kc, vc = (np.array(a, dtype=np.float64) for a in (M, z, kc, vc))
        B, Hq, d = q.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        out = np.empty((B, Hq, v.shape[2]))
        fold_at = seg_len - 2 if kind == "fold_early" else seg_len - 1
        for b in range(B):
            for j in range(Hkv):
                kc[b, j, pos], vc[b, j, pos] = k[b, j], v[b, j]
                if kind == "fold_first" and pos == fold_at:
                    M[b, j], z[b, j] = oracle.memory_update(kc[b, j], vc[b, j], M[b, j], z[b, j],
                                                            rule)
            for h in range(Hq):
                j = h % Hkv if kind == "gqa_modulo" else h // G
                n = pos if kind == "no_self" and pos > 0 else pos + 1
                s = kc[b, j, :n] @ q[b, h] / np.sqrt(d)
                w = np.exp(s - s.max())
                a_dot = w @ vc[b, j, :n] / w.sum()
                a_mem = oracle.memory_retrieval(q[b, h][None, :], M[b, j], z[b, j])[0]
                g = oracle.gate_weight(beta[h])
                out[b, h] = g * a_mem + (1 - g) * a_dot
            if kind != "fold_first" and pos == fold_at:
                for j in range(Hkv):
                    M[b, j], z[b, j] = oracle.memory_update(kc[b, j], vc[b, j], M[b, j], z[b, j],
                                                            rule)
        return out, M, z, kc, vc
    return step


@pytest.mark.parametrize("kind", ["no_self", "gqa_modulo", "fold_early", "fold_first"])
def test_planted_decode_mistakes_are_caught(rng, monkeypatch, kind):
    monkeypatch.setattr(oracle, "decode_step", _mutant(kind))
    with pytest.raises(AssertionError):
        test_decoding_a_stream_equals_the_forward(rng, "delta", 5)
