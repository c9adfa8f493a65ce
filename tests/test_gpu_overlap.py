"""The overlapped forward plan against the serial one, on the GPU.

With a workspace of the full size and a direct-form memory scan (seg_len < d,
or d_key != d_value), or the linear rule's affine form over at least 64
segments, on a large call (B*Hq*L*d >= 2^26), a forward call
starts segment 0's attention at once (from a snapshot of the initial state)
and runs the memory scan of the later segments on an auxiliary stream beside
the attention on the caller's stream. The arithmetic is the same kernels on
the same segments, so the results must equal the serial plan's (a workspace
one byte short of the full size) bit for bit: both key/value width layouts,
both rules, the training forward, an in-place state carry through calls
issued back to back with no synchronisation between them. One case checks the
overlapped result against the oracle on sampled segments, including segment
0 (the head start) and the first segment of each window.
"""

import sys

import pytest
import torch

from tests.parity import all_units, compare_units, random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MIN_ELEMS = 1 << 26  # B * Hq * L * d from which the overlapped plan runs


@pytest.fixture(scope="module")
def lib():
    import compressive_memory_transformers_amd as m
    return m


def _say(msg):
    print(f"[overlap] {msg}", flush=True)
    sys.stdout.flush()


def _full(lib, inp, seg_len, rule):
    B, Hq, L, d = inp["q"].shape
    full, _ = lib.workspace_size_kv(B, Hq, inp["k"].shape[1], L, d, inp["v"].shape[-1], seg_len,
                                    rule, inp["q"].dtype)
    return full


def _run(lib, inp, seg_len, rule, ws_bytes, lse=None):
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    res = lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"],
                      seg_len, rule, workspace=ws, lse=lse)
    torch.cuda.synchronize()
    return res


# (d_key, d_value, seg_len): seg_len < d, and d_key != d_value with long segments
@pytest.mark.parametrize("dk,dv,seg_len", [(128, 128, 64), (64, 128, 256)])
@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_overlapped_equals_serial(lib, rule, dk, dv, seg_len):
    _overlapped_equals_serial(lib, rule, dk, dv, seg_len)


def test_overlapped_linear_affine_equals_serial(lib):
    # the affine form's linear prefix over 128 segments (>= 64) of 256 tokens
    # also runs overlapped
    _overlapped_equals_serial(lib, "linear", 128, 128, 256)


def _overlapped_equals_serial(lib, rule, dk, dv, seg_len):
    B, Hq, Hkv = 2, 8, 2
    L = MIN_ELEMS // (B * Hq * dk)
    _say(f"bf16 B{B} Hq{Hq} Hkv{Hkv} d_key {dk} d_value {dv}, L {L}, seg_len {seg_len}, {rule}")
    inp = random_inputs(B, Hq, Hkv, L, dk, torch.bfloat16, DEV, seed=21, dv=dv)
    full = _full(lib, inp, seg_len, rule)
    a = _run(lib, inp, seg_len, rule, full - 1)  # serial, one window
    b = _run(lib, inp, seg_len, rule, full)      # overlapped
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_overlapped_train_forward_equals_serial(lib):
    B, Hq, Hkv, d, seg_len = 2, 8, 2, 64, 32
    L = MIN_ELEMS // (B * Hq * d)
    _say(f"training forward (lse), direct scan, delta, L {L}")
    inp = random_inputs(B, Hq, Hkv, L, d, torch.bfloat16, DEV, seed=22)
    full = _full(lib, inp, seg_len, "delta")
    outs = []
    for size in (full - 1, full):
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
        outs.append((*_run(lib, inp, seg_len, "delta", size, lse), lse))
    for x, y in zip(*outs):
        assert torch.equal(x, y)


def test_back_to_back_chained_calls(lib):
    """Three calls chained through an in-place state carry with no host
    synchronisation, each result copied by a torch kernel on the caller's
    stream right after its call: equal to the same chain run serially."""
    B, Hq, Hkv, d, seg_len = 1, 4, 2, 128, 64
    L = MIN_ELEMS // (B * Hq * d)
    _say(f"chained calls, in-place carry, L {L}, seg_len {seg_len}")
    inp = random_inputs(B, Hq, Hkv, L, d, torch.bfloat16, DEV, seed=23, m0_scale=0.2)
    full = _full(lib, inp, seg_len, "delta")

    def chain(size):
        ws = torch.empty(size, dtype=torch.uint8, device=DEV)
        M, z = inp["M0"].clone(), inp["z0"].clone()
        out = torch.empty((B, Hq, L, d), dtype=torch.bfloat16, device=DEV)
        seen = []
        for _ in range(3):
            lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], M, z, seg_len, "delta",
                        out=out, M_final=M, z_final=z, workspace=ws)
            seen.append((out.clone(), M.clone(), z.clone()))  # on the caller's stream
        torch.cuda.synchronize()
        return seen

    for x, y in zip(chain(full - 1), chain(full)):
        for s, t in zip(x, y):
            assert torch.equal(s, t)


def test_overlapped_parity_with_oracle(lib):
    B, Hq, Hkv, d, seg_len = 1, 4, 1, 128, 64
    L = MIN_ELEMS // (B * Hq * d)
    S = L // seg_len
    segs = [0, 1, 2, S // 4 - 1, S // 4, S // 2, S - 1]  # head start, both windows' edges
    _say(f"overlapped plan vs oracle, bf16 d128, {S} segments of {seg_len}, delta, GQA 4, "
         f"output segments {segs}")
    inp = random_inputs(B, Hq, Hkv, L, d, torch.bfloat16, DEV, seed=24)
    res = _run(lib, inp, seg_len, "delta", _full(lib, inp, seg_len, "delta"))
    eo, eM, ez = compare_units(inp, res, seg_len, "delta", all_units(B, Hkv), out_segments=segs)
    _say(f"errors out={eo:.3e} M={eM:.3e} z={ez:.3e}")
    assert max(eo, eM, ez) <= 2e-2
