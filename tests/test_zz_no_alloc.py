"""infini_attn_forward_noalloc, the forward whose workspace is the library's
per-GPU scratch array, against infini_attn_forward with a caller workspace of
the full size, through the C ABI. Two calls in a row, the second smaller than
the first, so the second starts from what the first left in the array; the
outputs must match bit for bit (the window plan does not change the
arithmetic). Each case prints what it runs before touching the GPU.
"""

import sys

import pytest
import torch

from tests.parity import random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    import compressive_memory_transformers_amd as m
    return m


def _say(msg):
    print(f"[noalloc] {msg}", flush=True)
    sys.stdout.flush()


def _both(lib, inp, seg_len, rule):
    args = [inp[n] for n in ("q", "k", "v", "beta", "M0", "z0")]
    ref = lib.forward(*args, seg_len, rule)
    out = torch.empty_like(ref[0])
    M = torch.empty_like(ref[1])
    z = torch.empty_like(ref[2])
    got = lib.forward_noalloc(*args, seg_len, rule, out=out, M_final=M, z_final=z)
    torch.cuda.synchronize()
    return ref, got


def _check(ref, got):
    for name, a, b in zip(("out", "M_final", "z_final"), ref, got):
        assert torch.equal(a, b), name


def test_two_calls_in_a_row_the_second_smaller(lib):
    import synth
    w = synth.WORKLOADS["llama3_8b"]
    B, Hq, Hkv, L, d = w.B, w.Hq, w.Hkv, w.L, w.d
    full, least = lib.workspace_size(B, Hq, Hkv, L, d, w.seg_len, "delta", torch.bfloat16)
    # the array holds the minimum but not the full size: the call walks windows
    assert least <= lib.binding.NOALLOC_SCRATCH_BYTES < full
    _say(f"call 1: llama3_8b (B{B} Hq{Hq} Hkv{Hkv} L{L} d{d} N{w.seg_len}, delta, bf16), "
         f"full workspace {full} vs scratch {lib.binding.NOALLOC_SCRATCH_BYTES}")
    inp = synth.make_inputs(w, DEV)
    ref, got = _both(lib, inp, w.seg_len, "delta")
    _check(ref, got)
    del inp, ref, got

    _say("call 2: B2 Hq8 Hkv2 L1000 d64 N100 (direct scan), linear, bf16, non-zero M0")
    inp = random_inputs(2, 8, 2, 1000, 64, torch.bfloat16, DEV, seed=31, m0_scale=0.3)
    ref, got = _both(lib, inp, 100, "linear")
    _check(ref, got)


def test_small_calls_and_in_place_carry(lib):
    cases = [
        # B, Hq, Hkv, L, d, seg_len, dtype, rule
        (1, 2, 2, 600, 32, 130, torch.float32, "delta"),   # affine form, ragged
        (1, 4, 4, 300, 64, 64, torch.bfloat16, "delta"),   # one pass with the state on chip
        (1, 1, 1, 1, 32, 16, torch.float32, "linear"),     # one token
    ]
    for B, Hq, Hkv, L, d, N, dt, rule in cases:
        _say(f"B{B} Hq{Hq} Hkv{Hkv} L{L} d{d} N{N} {dt} {rule}")
        inp = random_inputs(B, Hq, Hkv, L, d, dt, DEV, seed=L + d, m0_scale=0.2)
        ref, got = _both(lib, inp, N, rule)
        _check(ref, got)
    _say("in-place carry: M_final = M0, z_final = z0")
    inp = random_inputs(2, 4, 2, 500, 64, torch.bfloat16, DEV, seed=8, m0_scale=0.3)
    ref = lib.forward(*[inp[n] for n in ("q", "k", "v", "beta", "M0", "z0")], 96, "delta")
    M, z = inp["M0"].clone(), inp["z0"].clone()
    out = torch.empty_like(ref[0])
    lib.forward_noalloc(inp["q"], inp["k"], inp["v"], inp["beta"], M, z, 96, "delta", out=out,
                        M_final=M, z_final=z)
    torch.cuda.synchronize()
    _check(ref, (out, M, z))


def test_oversized_call_is_refused(lib):
    """A call whose minimum workspace exceeds the array is refused on the host."""
    _say("oversized: 4096 units of d = 128")
    q = torch.zeros(64, 64, 64, 128, dtype=torch.bfloat16, device=DEV)
    M0 = torch.zeros(64, 64, 128, 128, device=DEV)
    z0 = torch.ones(64, 64, 128, device=DEV)
    beta = torch.zeros(64, device=DEV)
    out = torch.empty_like(q)
    M, z = torch.empty_like(M0), torch.empty_like(z0)
    with pytest.raises(lib.InfiniAttnError) as e:
        lib.forward_noalloc(q, q.clone(), q.clone(), beta, M0, z0, 16, "delta", out=out,
                            M_final=M, z_final=z)
    assert e.value.status == 4
