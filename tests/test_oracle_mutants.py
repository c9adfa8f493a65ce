"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant replaces one oracle function (on the CPU, for the duration of one
test) with a plausible wrong version: a dropped term, a wrong sign or index, a
transposed operand, a step taken in the wrong order. The pins of
``test_oracle_pins.py`` are then run directly; the test passes when at least
one pin fails or raises.
"""

import inspect
import itertools
import math

import numpy as np
import pytest

import oracle.infini_attention as oi
import tests.test_oracle_pins as pins

_orig = {name: getattr(oi, name) for name in
         ("feature_map", "local_causal_attention", "memory_retrieval",
          "memory_update", "forward", "gate_weight")}


def _attn(scale_fn=math.sqrt, diag=True):
    def f(q, k, v):
        n, d = q.shape
        s = (q @ k.T) / scale_fn(d)
        s = np.where(np.triu(np.ones((n, n), bool), k=1 if diag else 0), -np.inf, s)
        s = s - s.max(axis=1, keepdims=True)
        w = np.exp(s)
        return (w @ v) / w.sum(axis=1, keepdims=True)
    return f


def _update(kind):
    def f(k, v, M, z, rule):
        if rule not in oi.RULES:
            raise ValueError(rule)
        sk = _orig["feature_map"](k)
        if rule == "linear":
            M_new = M + (v.T @ sk if kind == "transposed" and v.shape[1] == sk.shape[1]
                         else sk.T @ v)
        else:
            zz = z + sk.sum(0) if kind == "new_z" else z
            pred = sk @ M
            if kind != "no_denominator":
                pred = pred / (sk @ zz)[:, None]
            r = v + pred if kind == "sign" else v - pred
            M_new = M + sk.T @ r
        z_new = z if kind == "no_z" else z + sk.sum(0)
        return M_new, z_new
    return f


def _retrieval(kind):
    def f(q, M, z):
        sq = _orig["feature_map"](q)
        if kind == "transposed":
            return (sq @ M.T) / (sq @ z)[:, None]
        if kind == "elementwise_den":
            return (sq @ M) / (sq * z).sum(1, keepdims=True).clip(min=1e-300) ** 0.5
        if kind == "raw_query":
            return (q @ M) / (sq @ z)[:, None]
        raise AssertionError(kind)
    return f


def _forward_update_first(q, k, v, beta, M0, z0, seg_len, rule, units=None, out_segments=None):
    q, k, v, beta, M0, z0 = (np.asarray(a, dtype=np.float64) for a in (q, k, v, beta, M0, z0))
    B, Hq, L, _ = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.full((B, Hq, L, v.shape[3]), np.nan)
    Mf, zf = np.full(M0.shape, np.nan), np.full(z0.shape, np.nan)
    for b, j in ([(b, j) for b in range(B) for j in range(Hkv)] if units is None else units):
        M, z = M0[b, j].copy(), z0[b, j].copy()
        for s in range(oi.num_segments(L, seg_len)):
            t0, t1 = s * seg_len, min((s + 1) * seg_len, L)
            M, z = oi.memory_update(k[b, j, t0:t1], v[b, j, t0:t1], M, z, rule)
            if out_segments is None or s in out_segments:
                for h in range(j * G, (j + 1) * G):
                    g = oi.gate_weight(beta[h])
                    out[b, h, t0:t1] = (g * oi.memory_retrieval(q[b, h, t0:t1], M, z)
                                        + (1 - g) * oi.local_causal_attention(
                                            q[b, h, t0:t1], k[b, j, t0:t1], v[b, j, t0:t1]))
        Mf[b, j], zf[b, j] = M, z
    return out, Mf, zf


MUTANTS = {
    "elu_without_plus_one": ("feature_map", lambda x: np.where(np.asarray(x, float) > 0, x, np.expm1(np.minimum(x, 0.0)) + 1e-3)),
    "sigma_is_x_plus_one": ("feature_map", lambda x: np.asarray(x, float) + 1.0),
    "sigma_is_relu": ("feature_map", lambda x: np.maximum(np.asarray(x, float), 0.0) + 1e-9),
    "mask_hides_diagonal": ("local_causal_attention", _attn(diag=False)),
    "scale_by_d": ("local_causal_attention", _attn(scale_fn=float)),
    "no_scale": ("local_causal_attention", _attn(scale_fn=lambda d: 1.0)),
    "retrieval_transposed_memory": ("memory_retrieval", _retrieval("transposed")),
    "retrieval_wrong_denominator": ("memory_retrieval", _retrieval("elementwise_den")),
    "retrieval_without_sigma": ("memory_retrieval", _retrieval("raw_query")),
    "delta_residual_sign": ("memory_update", _update("sign")),
    "delta_uses_new_z": ("memory_update", _update("new_z")),
    "delta_without_denominator": ("memory_update", _update("no_denominator")),
    "z_not_updated": ("memory_update", _update("no_z")),
    "linear_update_transposed": ("memory_update", _update("transposed")),
    "gate_swapped": ("gate_weight", lambda beta: 1.0 - _orig["gate_weight"](beta)),
    "update_before_retrieval": ("forward", _forward_update_first),
}


def _pin_calls():
    """(name, function, kwargs) for every pin, parametrisations expanded."""
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = {}
        for mark in getattr(fn, "pytestmark", []):
            if mark.name == "parametrize":
                argnames, values = mark.args[0], mark.args[1]
                argnames = [a.strip() for a in argnames.split(",")]
                params[tuple(argnames)] = values
        combos = [{}]
        for argnames, values in params.items():
            new = []
            for base, val in itertools.product(combos, values):
                val = val if len(argnames) > 1 else (val,)
                new.append({**base, **dict(zip(argnames, val))})
            combos = new
        for kw in combos:
            calls.append((name, fn, kw))
    return calls


def _run_pins():
    failed = []
    for name, fn, kw in _pin_calls():
        sig = inspect.signature(fn)
        if "rng" in sig.parameters:
            kw = {**kw, "rng": np.random.default_rng(12345)}
        try:
            with np.errstate(all="ignore"):
                fn(**kw)
        except (KeyboardInterrupt, SystemExit):
            raise
        except BaseException:  # a failed check (pytest's own included) or a crash
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(monkeypatch, mutant):
    target, fake = MUTANTS[mutant]
    monkeypatch.setattr(oi, target, fake)
    monkeypatch.setattr(pins, target, fake, raising=False)
    failed = _run_pins()
    assert failed, f"no pin catches the planted mistake {mutant!r}"
