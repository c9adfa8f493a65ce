"""The forward captured into a HIP graph and replayed, on the GPU.

The library allocates nothing, synchronises nothing and clears no memory with
hipMemsetAsync inside a call, so a call can be captured into a graph (torch's
CUDAGraph over the HIP runtime) and replayed. Each case captures one call,
then replays it three times with eager work between the replays (the outputs
overwritten, another forward call on other inputs through another workspace)
and checks every replay against the eager call bit for bit: the one-pass plan
(short segments), the serial split plan (the affine form), the overlapped
plan (a direct scan on an auxiliary stream, forked from and joined back into
the captured stream by events) and the fp32 path. The streaming decode
step is captured too: one step at a fixed position, and a whole segment of
steps (each with its own position, the fold into the state at the last) as
one graph, replayed from reset state buffers.
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
    print(f"[graph] {msg}", flush=True)
    sys.stdout.flush()


def _workspace(lib, inp, seg_len, rule):
    B, Hq, L, d = inp["q"].shape
    full, _ = lib.workspace_size_kv(B, Hq, inp["k"].shape[1], L, d, inp["v"].shape[-1],
                                    seg_len, rule, inp["q"].dtype)
    return torch.empty(full, dtype=torch.uint8, device=DEV)


def _call(lib, inp, seg_len, rule, out, M, z, ws, stream):
    lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"], seg_len, rule,
                out=out, M_final=M, z_final=z, workspace=ws, stream=stream)


CASES = [
    # (B, Hq, Hkv, L, d, seg_len, rule, dtype): the plan each one takes
    (2, 4, 4, 512, 64, 64, "delta", torch.bfloat16),        # one pass
    (1, 8, 2, 4096, 128, 1024, "delta", torch.bfloat16),    # serial split, affine form
    (2, 8, 2, 32768, 128, 64, "linear", torch.bfloat16),    # overlapped, direct scan
    (1, 2, 2, 64, 32, 16, "linear", torch.float32),         # fp32 path
]


@pytest.mark.parametrize("case", CASES, ids=["one_pass", "serial_affine", "overlapped",
                                             "fp32"])
def test_graph_replays_equal_eager(lib, case):
    B, Hq, Hkv, L, d, N, rule, dt = case
    _say(f"B{B} Hq{Hq} Hkv{Hkv} L{L} d{d} N{N} {rule} {dt}")
    inp = random_inputs(B, Hq, Hkv, L, d, dt, DEV, seed=31)
    other = random_inputs(B, Hq, Hkv, L, d, dt, DEV, seed=32)
    ws = _workspace(lib, inp, N, rule)
    ws2 = _workspace(lib, inp, N, rule)
    out = torch.empty((B, Hq, L, d), dtype=dt, device=DEV)
    M = torch.empty_like(inp["M0"])
    z = torch.empty_like(inp["z0"])
    cur = torch.cuda.current_stream(DEV)
    _call(lib, inp, N, rule, out, M, z, ws, cur)
    torch.cuda.synchronize()
    ref = (out.clone(), M.clone(), z.clone())

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(lib, inp, N, rule, out, M, z, ws, torch.cuda.current_stream(DEV))
    out2 = torch.empty_like(out)
    M2, z2 = torch.empty_like(M), torch.empty_like(z)
    for rep in range(3):
        # eager work between the replays: the outputs overwritten, and
        # another call on other inputs through another workspace
        out.fill_(float("nan"))
        M.fill_(float("nan"))
        z.fill_(float("nan"))
        _call(lib, other, N, rule, out2, M2, z2, ws2, cur)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"replay {rep}")
        for got, want in zip((out, M, z), ref):
            assert torch.equal(got, want), f"replay {rep} differs from the eager call"
    del g


def test_decode_graphs_replay_equal_eager(lib):
    # a decode step at a fixed position, and a whole segment of steps (each
    # with its own position, the fold into the state at the last) as one
    # graph, both replayed from reset state buffers
    B, Hq, Hkv, d, N, rule = 2, 8, 2, 128, 64, "delta"
    _say(f"decode B{B} Hq{Hq} Hkv{Hkv} d{d} N{N} {rule}")
    g = torch.Generator(device="cpu").manual_seed(41)
    mk = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).to(DEV)
    q = [mk(B, Hq, d) for _ in range(N)]
    k = [mk(B, Hkv, d) for _ in range(N)]
    v = [mk(B, Hkv, d) for _ in range(N)]
    beta = torch.randn(Hq, generator=g).to(DEV)
    kc0 = torch.zeros(B, Hkv, N, d, dtype=torch.bfloat16, device=DEV)
    M0 = (0.1 * torch.randn(B, Hkv, d, d, generator=g)).to(DEV)
    z0 = (0.5 + torch.rand(B, Hkv, d, generator=g)).to(DEV)
    ws = torch.empty(lib.decode_workspace_size(B, Hq, Hkv, d, N, rule, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)
    kc, vc = kc0.clone(), kc0.clone()
    M, z = M0.clone(), z0.clone()
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=DEV)
    outs = torch.empty(N, B, Hq, d, dtype=torch.bfloat16, device=DEV)

    def segment(stream):
        for pos in range(N):
            lib.decode_step(q[pos], k[pos], v[pos], beta, kc, vc, M, z, pos, rule, out=out,
                            workspace=ws, stream=stream)
            outs[pos].copy_(out)

    def reset():
        kc.copy_(kc0)
        vc.copy_(kc0)
        M.copy_(M0)
        z.copy_(z0)
        outs.fill_(float("nan"))

    cur = torch.cuda.current_stream(DEV)
    segment(cur)
    torch.cuda.synchronize()
    ref = (outs.clone(), kc.clone(), vc.clone(), M.clone(), z.clone())
    reset()
    gseg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gseg):
        segment(torch.cuda.current_stream(DEV))
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        gseg.replay()
        torch.cuda.synchronize()
        _say(f"segment replay {rep}")
        for got, want in zip((outs, kc, vc, M, z), ref):
            assert torch.equal(got, want), f"segment replay {rep} differs from the eager steps"

    # one step at a full cache (no fold), against an eager call of it
    pos = N - 2
    lib.decode_step(q[pos], k[pos], v[pos], beta, kc, vc, M, z, pos, rule, out=out,
                    workspace=ws, stream=cur)
    torch.cuda.synchronize()
    want = out.clone()
    gstep = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gstep):
        lib.decode_step(q[pos], k[pos], v[pos], beta, kc, vc, M, z, pos, rule, out=out,
                        workspace=ws, stream=torch.cuda.current_stream(DEV))
    kc2, vc2, M2, z2 = kc0.clone(), kc0.clone(), M0.clone(), z0.clone()
    ws2, out2 = torch.empty_like(ws), torch.empty_like(out)
    for rep in range(3):
        out.fill_(float("nan"))
        # eager work between: a step on other buffers
        lib.decode_step(q[1], k[1], v[1], beta, kc2, vc2, M2, z2, 3, rule, out=out2,
                        workspace=ws2, stream=cur)
        torch.cuda.synchronize()
        gstep.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"step replay {rep} differs from the eager step"
    del gseg, gstep
