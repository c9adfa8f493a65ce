"""Very long segments: the forward with 100000-token segments against the
row-restricted oracle (oracle.forward_rows) on sampled rows of every segment
(first, last, the segment boundary's neighbours and seeded random rows),
and the final state in full. Each case prints what it runs before touching
the GPU."""

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
    print(f"[long] {msg}", flush=True)
    sys.stdout.flush()


CASES = [
    # B, Hq, Hkv, L, d, seg_len
    (1, 2, 1, 200000, 128, 100000),  # two full 100k-token segments, two heads on one KV head
    (1, 1, 1, 150000, 64, 100000),   # a full and a ragged (50k) segment
]


@pytest.mark.parametrize("case", CASES, ids=["2x100k-d128-gqa2", "100k+50k-d64"])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_long_segments_match_the_oracle_on_sampled_rows(lib, case, rule):
    B, Hq, Hkv, L, d, N = case
    _say(f"{case} {rule}")
    inp = random_inputs(B, Hq, Hkv, L, d, torch.bfloat16, DEV, seed=L + d, m0_scale=0.3)
    out, M, z = lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"], N,
                            rule)
    torch.cuda.synchronize()
    g = np.random.default_rng(L)
    rows = sorted({0, 1, N - 1, N, N + 1, L - 1, *g.integers(0, L, 10).tolist()})
    f = {k: synth.to_f64(v) for k, v in inp.items()}
    ref, rM, rz = oracle.forward_rows(f["q"], f["k"], f["v"], f["beta"], f["M0"], f["z0"], N,
                                      rule, rows)
    got = synth.to_f64(out)[:, :, rows]
    errs = dict(out=oracle.slice_errors(got, ref), M=oracle.slice_errors(synth.to_f64(M), rM),
                z=oracle.slice_errors(synth.to_f64(z), rz, elementwise=True))
    _say("errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    tol = tolerance(torch.bfloat16)
    assert all(v <= tol for v in errs.values()), (errs, tol)
