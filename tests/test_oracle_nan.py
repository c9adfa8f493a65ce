"""A NaN stays inside the slices it touches (oracle, CPU).

"Infini-Attention" (AI Wiki), "Why is the memory footprint bounded?": each
stream carries only its own (M, z); a (batch, KV head) unit never reads
another unit's tokens or state. And "What happens inside the Infini-attention
block?": row t of A_dot reads keys 0..t of its segment only, and A_mem reads
the state left by the earlier segments. So a NaN key row at position t of
segment s of one unit makes exactly these entries NaN: that unit's output rows
t.. of segment s and every row of the later segments (through M and z), for
each query head of its group, and its final state. A NaN query row makes only
its own output row NaN. Everything else is bit for bit the result without the
NaN.
"""

import numpy as np
import pytest

import oracle


def _inputs(seed, B=2, Hq=4, Hkv=2, L=50, dk=8, dv=8):
    rng = np.random.default_rng(seed)
    return dict(q=rng.standard_normal((B, Hq, L, dk)), k=rng.standard_normal((B, Hkv, L, dk)),
                v=rng.standard_normal((B, Hkv, L, dv)), beta=rng.standard_normal(Hq),
                M0=0.1 * rng.standard_normal((B, Hkv, dk, dv)),
                z0=1.0 + rng.random((B, Hkv, dk)))


def _run(inp, N, rule):
    return oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"], N, rule)


@pytest.mark.parametrize("rule", ["linear", "delta"])
@pytest.mark.parametrize("dv", [8, 12])
def test_nan_key_row_is_confined_to_its_unit(rule, dv):
    N, tk = 16, 21                       # key row 21: segment 1, its 6th row
    inp = _inputs(3, dv=dv)
    clean = _run(inp, N, rule)
    inp["k"][1, 0, tk, :] = np.nan
    out, M, z = _run(inp, N, rule)
    G = 2
    rows = np.zeros(out.shape[:3], dtype=bool)
    rows[1, 0:G, tk:] = True             # rows tk.. of its segment, then all later rows
    assert np.array_equal(np.isnan(out), np.broadcast_to(rows[..., None], out.shape))
    assert np.array_equal(out[~np.isnan(out)], clean[0][~np.isnan(out)])
    assert np.isnan(M[1, 0]).all() and np.isnan(z[1, 0]).all()
    others = [(0, 0), (0, 1), (1, 1)]
    for b, j in others:
        assert np.array_equal(M[b, j], clean[1][b, j]) and np.array_equal(z[b, j], clean[2][b, j])


def test_nan_key_row_leaves_earlier_rows_of_its_segment_alone():
    N, tk = 16, 20                       # row 20 of segment 1 (rows 16..31)
    inp = _inputs(5)
    clean = _run(inp, N, "delta")
    inp["k"][0, 1, tk + 3, :] = np.nan   # key row 23: rows 16..22 never see it
    out, _, _ = _run(inp, N, "delta")
    rows = np.isnan(out[0, 2]).any(axis=-1)
    assert not rows[:tk + 3].any() and rows[tk + 3:].all()
    assert np.array_equal(out[0, 2, :tk + 3], clean[0][0, 2, :tk + 3])


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_nan_query_row_is_confined_to_its_row(rule):
    N, tq = 16, 7
    inp = _inputs(4)
    clean = _run(inp, N, rule)
    inp["q"][0, 1, tq, :] = np.nan
    out, M, z = _run(inp, N, rule)
    bad = np.isnan(out)
    assert bad[0, 1, tq].all() and bad.sum() == out.shape[-1]
    assert np.array_equal(out[~bad], clean[0][~bad])
    # the query never enters the state
    assert np.array_equal(M, clean[1]) and np.array_equal(z, clean[2])
