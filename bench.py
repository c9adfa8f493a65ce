#!/usr/bin/env python3
"""Throughput of the Infini-attention block forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

One step is one infini_attn_forward call over the whole workload (every
segment, every head): the memory scan and the fused local-attention /
retrieval / gate kernel, on synthetic Gaussian inputs already resident in HBM.
W untimed steps, then K timed steps between two device synchronisations: the
step captured once into a HIP graph and replayed K times (the same kernels on
the same buffers, without the host's per-launch work between them; the mean
of K eager calls is reported beside it, and per-step and per-phase HIP events
come from the eager calls).
Prints one JSON line: tokens/s (B*L / step time), TFLOP/s and its fraction of
the bf16 MFMA peak, the roofline record of the dominant kernel (timed with HIP
events on the stream it runs on) and the fp64 CPU oracle's rate on a bounded
sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "Infini-attn fwd tokens/s + TFLOP/s (% bf16 MFMA peak), 1×MI355X"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the sources that decide the dominant kernel's memory traffic: the attention
# kernel of the split plan, or the one-pass fused kernel
_CSRC = os.path.join(ROOT, "compressive_memory_transformers_amd", "csrc")
ATTN_SOURCES = [os.path.join(_CSRC, f) for f in ("attn.hip", "lds_tile.hpp", "common.hpp")]
FUSED_SOURCES = [os.path.join(_CSRC, f) for f in ("fused.hip", "lds_tile.hpp", "common.hpp")]


def attn_kernel_bytes(w):
    """Algorithmic HBM bytes of the attention kernel in one call: Q and out
    once, K and V once, and the per-segment state it reads (M^T in the element
    type and z in float, per KV head and segment), beta once."""
    e = 4 if w.dtype == "f32" else 2
    d, dv = w.d, w.d_value
    return (e * w.L * w.B * ((d + dv) * w.Hq + (d + dv) * w.Hkv)
            + w.B * w.Hkv * w.segments * (d * dv * e + 4 * d) + 4 * w.Hq)


def attn_kernel_flops(w):
    """Algorithmic matrix-product FLOPs of the attention kernel in one call:
    per (query head, token) 2d(N+1) for the causal QK^T and PV (diagonal
    counted) and 2d^2 for sigma(Q) M, summed exactly over segments; with a
    value width dv, (d + dv)(N+1) and 2 d dv."""
    d, dv = w.d, w.d_value
    total = 0
    for s in range(w.segments):
        n = min(w.seg_len, w.L - s * w.seg_len)
        total += (d + dv) * n * (n + 1) + 2 * n * d * dv
    return w.B * w.Hq * total


def uses_fused_plan(w):
    """Whether the library runs this workload's forward as the one-pass fused
    kernel (the condition the library's plan applies: bf16, d_key = d_value
    in {64, 128}, as many query as KV heads, segments no longer than d)."""
    return (w.dtype == "bf16" and w.d == w.d_value and w.d in (64, 128) and w.Hq == w.Hkv
            and min(w.seg_len, w.L) <= w.d)


def source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(w, rule):
    """HBM bytes per launch of the workload's dominant kernel from committed
    rocprofv3 counters, or None when there are none for this workload and
    configuration or the kernel's sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(w.name)
    except (OSError, ValueError):
        return None
    srcs = FUSED_SOURCES if uses_fused_plan(w) else ATTN_SOURCES
    if (not rec or rec.get("hashed_sources") != [os.path.relpath(p, ROOT) for p in srcs]
            or rec.get("source_sha256_16") != source_hash(srcs)
            or rec.get("seg_len") != w.seg_len or rec.get("rule") != rule):
        return None
    return rec.get("bytes_per_launch")


def _oracle_unit(task):
    """One (batch, KV head) unit of the workload through the fp64 oracle in a
    pool worker with one BLAS thread; returns the oracle's run time."""
    import threadpoolctl

    import oracle

    w, rule, b, j = task
    with threadpoolctl.threadpool_limits(1):
        u = synth.make_unit_inputs(w, b, j)
        t0 = time.perf_counter()
        oracle.forward(u["q"], u["k"], u["v"], u["beta"], u["M0"], u["z0"], w.seg_len, rule)
        return time.perf_counter() - t0


def cpu_pool(procs):
    """A pool of `procs` worker processes, forked before this process touches
    the GPU (the workers only run the CPU oracle)."""
    import multiprocessing
    return multiprocessing.get_context("fork").Pool(procs)


def cpu_baseline(pool, procs, w, rule, target_s):
    """The fp64 oracle, as it is, on whole (batch, KV head) units of the same
    workload (inputs drawn on the CPU from the same per-slice seeds), one unit
    per worker process, in rounds of `procs` units until about target_s
    seconds of wall time have run (or every unit is done)."""
    order = [(b, j) for b in range(w.B) for j in range(w.Hkv)]
    done, t0 = 0, time.perf_counter()
    while done < len(order):
        batch = order[done:done + procs]
        pool.map(_oracle_unit, [(w, rule, b, j) for b, j in batch], chunksize=1)
        done += len(batch)
        if time.perf_counter() - t0 >= target_s:
            break
    wall = time.perf_counter() - t0
    G = w.Hq // w.Hkv
    tokens = w.B * w.L * done / len(order)
    return {
        "value": tokens / wall,
        "unit": "tokens/s",
        "cores": int(min(procs, done)),
        "kind": "oracle",
        "sample": (f"{done} of {len(order)} (batch, KV head) units, each {G} query heads x "
                   f"{w.segments} segments of {w.seg_len}, one unit per process on "
                   f"{min(procs, done)} processes with one BLAS thread each; fp64 numpy, "
                   f"{wall:.1f} s wall; value = B*L*{done}/{len(order)} tokens / wall time"),
    }


def gpu_sclk_mhz():
    """The current shader clock of GPU 0 in MHz from rocm-smi, or None."""
    import re
    import subprocess
    try:
        txt = subprocess.run(["rocm-smi", "-d", "0", "--showclocks"], capture_output=True,
                             text=True, timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    m = re.search(r"sclk[^\n]*?\((\d+)\s*Mhz\)", txt, flags=re.I)
    return int(m.group(1)) if m else None


# The pages' own numbers for Infini-attention models, for context only: none
# comes with hardware or a throughput ("Infini-Attention" (AI Wiki), "Results
# at a glance" and "Can Infini-attention retrieve a passkey at one million
# tokens?"; "Hugging Face Infini-Attention Reproduction Analysis", "Weight
# Decay and Rollouts").
PAGES_CONTEXT = {
    "passkey": "1B model, passkey retrieval up to 1M tokens, about 100% after fine-tuning",
    "booksum": "8B model, book summarisation over 500K tokens, ROUGE 40.0 / 8.8 / 17.9",
    "hf_reproduction": "200M Llama and Llama 3 8B, 64-token segments x 16 rollouts",
    "hardware": "not stated on the pages; no throughput is published",
}


def decode_bytes(w, pos):
    """Algorithmic HBM bytes of one decode step at position pos: the cached
    keys and values of rows 0..pos once, the float state once, q and out of
    the token, its key and value written into the caches."""
    e = 4 if w.dtype == "f32" else 2
    units = w.B * w.Hkv
    return (units * (2 * (pos + 1) * w.d * e + 4 * (w.d * w.d + w.d))
            + 2 * w.B * w.Hq * w.d * e + 2 * units * w.d * e)


def bench_decode(lib, w, rule, dev, args):
    """The streaming decode step over one full segment of the workload's
    shape: seg_len steps, positions 0 .. seg_len-1, the last one folding the
    segment into the state. Every step takes one token per (batch, head)."""
    import torch

    g = torch.Generator(device="cpu").manual_seed(7)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    N, d = w.seg_len, w.d
    mk = lambda *s: torch.randn(*s, generator=g, dtype=torch.float32).to(dt).to(dev)
    q = [mk(w.B, w.Hq, d) for _ in range(8)]
    k = [mk(w.B, w.Hkv, d) for _ in range(8)]
    v = [mk(w.B, w.Hkv, d) for _ in range(8)]
    beta = torch.randn(w.Hq, generator=g).to(dev)
    kc = torch.zeros(w.B, w.Hkv, N, d, dtype=dt, device=dev)
    vc = torch.zeros_like(kc)
    M = torch.zeros(w.B, w.Hkv, d, d, device=dev)
    z = torch.full((w.B, w.Hkv, d), 1e-6, device=dev)
    out = torch.empty_like(q[0])
    ws = torch.empty(lib.decode_workspace_size(w.B, w.Hq, w.Hkv, d, N, rule, dt),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(pos):
        lib.decode_step(q[pos % 8], k[pos % 8], v[pos % 8], beta, kc, vc, M, z, pos, rule,
                        out=out, workspace=ws, stream=stream)

    for pos in range(min(args.warmup, N)):
        step(pos)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for pos in range(N):
        step(pos)
    e1.record(stream)
    torch.cuda.synchronize()
    seg_ms = e0.elapsed_time(e1)
    # one step at a full cache without the fold (pos = N - 2), repeated
    reps = 50
    e0.record(stream)
    for _ in range(reps):
        step(N - 2)
    e1.record(stream)
    torch.cuda.synchronize()
    full_us = e0.elapsed_time(e1) / reps * 1e3
    # the segment again, captured into one HIP graph and replayed, as a
    # serving loop would run it: its N steps, each with its own position,
    # the fold at the end. (A graph of the single full-cache step replays
    # slower than its two eager launches, about 29 against 17 us, so that
    # figure stays eager.)
    seg_ms_eager, graph_error = seg_ms, None
    if args.graph:
        try:
            gseg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gseg):
                cap = torch.cuda.current_stream(dev)
                for pos in range(N):
                    lib.decode_step(q[pos % 8], k[pos % 8], v[pos % 8], beta, kc, vc, M, z, pos,
                                    rule, out=out, workspace=ws, stream=cap)
        except RuntimeError as e:  # capture refused: the eager timing stands
            gseg = None
            graph_error = str(e)[:200]
            torch.cuda.synchronize()
        if gseg is not None:
            gseg.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            gseg.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            seg_ms = e0.elapsed_time(e1)
            del gseg
    gbs = decode_bytes(w, N - 2) / (full_us * 1e-6) / 1e9
    return {
        "metric": "Infini-attn streaming decode tokens/s, 1xMI355X",
        "value": w.B * N / (seg_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": N,
        "warmup": min(args.warmup, N),
        "ms_per_step": seg_ms / N,
        "timing": ("the segment's steps as one HIP graph, replayed" if graph_error is None
                   and args.graph else "eager launches"),
        "eager_segment_ms": seg_ms_eager,
        "graph_error": graph_error,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian q/k/v; zero initial state)",
        "config": {"workload": w.name + "/decode", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": d,
                   "seg_len": N, "rule": rule, "tokens_per_step": w.B},
        "segment_ms": seg_ms,
        "full_cache_step_us": full_us,
        "roofline": {"kernel": "decode step at a full cache (partial + combine)", "bound": "hbm",
                     "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": decode_bytes(w, N - 2)},
        "cpu_baseline": None,
    }


def bwd_flops(w, rule):
    """Algorithmic matrix-product FLOPs of one backward call: per (query head,
    segment of n rows) 5 causal products of d n (n + 1) each for the local
    attention (S, dP, dV, dK, dQ); per query row 6 d^2 for the retrieval
    (sigma(Q) M, dn M^T, sigma(Q)^T dn); per key row 4 d^2 for the linear
    update's (Phi dM, V dM^T), 10 d^2 for the delta rule's (also Phi M,
    dP M^T and A_s); 2 d^3 per (unit, segment) for the delta chain."""
    d = w.d
    local = 0
    for s_ in range(w.segments):
        n = min(w.seg_len, w.L - s_ * w.seg_len)
        local += 5 * d * n * (n + 1)
    local *= w.B * w.Hq
    retr = 6 * d * d * w.B * w.Hq * w.L
    upd = (10 if rule == "delta" else 4) * d * d * w.B * w.Hkv * w.L
    chain = (2 * d ** 3 * w.B * w.Hkv * w.segments) if rule == "delta" else 0
    return local + retr + upd + chain, local


def bench_backward(lib, w, rule, dev, args):
    """The backward pass over the whole workload: one infini_attn_backward
    call per step, with the forward's out and lse (one training forward)
    and a random d_out resident in HBM; no gradient on the final state."""
    import torch

    inp = synth.make_inputs(w, dev)
    dt = inp["q"].dtype
    g = torch.Generator(device="cpu").manual_seed(9)
    d_out = torch.randn(w.B, w.Hq, w.L, w.d, generator=g).to(dt).to(dev)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):  # the second call is timed (the first one warms up)
        e0.record(stream)
        out, _, _, lse = lib.forward_train(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"],
                                           inp["z0"], w.seg_len, rule)
        e1.record(stream)
        torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1)
    ws = torch.empty(lib.backward_workspace_size(w.B, w.Hq, w.Hkv, w.L, w.d, w.seg_len, rule, dt),
                     dtype=torch.uint8, device=dev)

    def step():
        return lib.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"],
                            w.seg_len, rule, out, lse, d_out, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        grads = step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    finite = all(bool(torch.isfinite(x).all()) for x in grads[:4])
    flops, local = bwd_flops(w, rule)
    peak = PEAK_TFLOPS["bf16" if w.dtype == "bf16" else "f32"]
    tf = flops / (ms * 1e-3) / 1e12
    return {
        "metric": "Infini-attn backward tokens/s + TFLOP/s, 1xMI355X",
        "value": w.B * w.L / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian Q/K/V and d_out in HBM; random beta; M0 = 0, "
                "z0 = 1e-6)",
        "config": {"workload": w.name + "/backward", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "L": w.L, "d": w.d, "seg_len": w.seg_len, "rule": rule},
        "forward_train_ms": fwd_ms,
        "gradients_finite": finite,
        "tflops": tf,
        "roofline": {"kernel": "whole backward call (local-attention gradients dominate)",
                     "bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                     "frac": tf / peak, "traffic": None,
                     "algorithmic_flop_per_launch": flops,
                     "local_attention_flop_per_launch": local},
        "cpu_baseline": None,
    }


BLOCK_D_MODEL = {"llama3_8b": 4096, "hf_repro": 1024, "tiny": 64, "long_stream": 2048,
                 "small_segment": 4096, "long_segment": 2048}


def bench_block(lib, w, rule, dev, args):
    """The block with its projections (Q/K/V and output, random weights of the
    layer's shape): one infini_attn_block_forward call per step, x and the
    weights resident in HBM. The roofline is the input projection's (the
    kernel with the most work), timed with HIP events on its own stream."""
    import torch

    dm = BLOCK_D_MODEL[w.name]
    inp = synth.make_block_inputs(w.B, w.L, dm, w.Hq, w.Hkv, w.d, torch.bfloat16, device=dev,
                                  seed=w.seed, z0=w.z0)
    stream = torch.cuda.current_stream(dev)
    ws = torch.empty(lib.block_workspace_size(w.B, w.L, dm, w.Hq, w.Hkv, w.d, w.seg_len, rule),
                     dtype=torch.uint8, device=dev)
    args_ = [inp[k] for k in ("x", "w_qkv", "w_o", "beta", "M0", "z0")]

    def step(events=None):
        return lib.block_forward(*args_, w.seg_len, rule, w.Hq, w.Hkv, workspace=ws,
                                 stream=stream, events=events)

    for _ in range(args.warmup):
        step()
    # per-phase events for every timed step; recorded once first so each
    # underlying HIP event exists before the library records it
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for row in ev:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        y, _, _ = step(ev[i])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    phases = [sum(row[p].elapsed_time(row[p + 1]) for row in ev) / args.steps for p in range(3)]
    finite = bool(torch.isfinite(y).all())
    M = w.B * w.L
    nqkv = (w.Hq + 2 * w.Hkv) * w.d
    qkv_flop = 2 * M * dm * nqkv
    o_flop = 2 * M * w.Hq * w.d * dm
    flops = synth.block_flops(w.B, w.L, dm, w.Hq, w.Hkv, w.d, w.seg_len, rule)
    peak = PEAK_TFLOPS["bf16"]
    tf = flops / (ms * 1e-3) / 1e12
    ach = qkv_flop / (phases[0] * 1e-3) / 1e12
    return {
        "metric": "Infini-attn block with Q/K/V and output projections, tokens/s + TFLOP/s, "
                  "1xMI355X",
        "value": M / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian x, weights N(0, 1/fan_in), random beta; "
                f"M0 = 0, z0 = {w.z0})",
        "config": {"workload": w.name + "/block", "B": w.B, "L": w.L, "d_model": dm,
                   "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "seg_len": w.seg_len, "rule": rule},
        "output_finite": finite,
        "tflops": tf,
        "phase_ms": {"qkv_projection": phases[0], "block": phases[1],
                     "out_projection": phases[2]},
        "projection_tflops": {"qkv": ach, "out": o_flop / (phases[2] * 1e-3) / 1e12},
        "roofline": {"kernel": "proj_kernel (Q/K/V projection, heads split in the epilogue)",
                     "bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                     "frac": ach / peak, "traffic": None,
                     "algorithmic_flop_per_launch": qkv_flop},
        "cpu_baseline": None,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--rule", default=None, choices=["linear", "delta"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target length of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="forward", choices=["forward", "decode", "backward", "block"],
                    help="forward: the block forward over the workload (default); decode: "
                         "the streaming decode step over one full segment of it; backward: "
                         "the gradients of the block over the workload; block: the block "
                         "with its Q/K/V and output projections over the workload")
    ap.add_argument("--seg-len", type=int, default=0,
                    help="override the workload's segment length (same L; a sweep point)")
    ap.add_argument("--plan", default="overlapped", choices=["overlapped", "serial"],
                    help="overlapped: the full workspace (the scan beside the attention); "
                         "serial: one byte less (scan, then attention, on one stream)")
    ap.add_argument("--cold", type=int, default=5, metavar="N",
                    help="also time N steps each after flushing the caches with a 512 MiB "
                         "device copy outside the timed events (0: skip)")
    ap.add_argument("--sclk-samples", type=int, default=3, metavar="N",
                    help="sample the shader clock N times while steps run (0: skip)")
    ap.add_argument("--cpu-procs", type=int, default=16,
                    help="worker processes of the CPU oracle (at most the host's CPUs)")
    ap.add_argument("--graph", type=int, default=1, choices=[0, 1],
                    help="1 (forward mode): ms_per_step and value from replays of a HIP graph "
                         "captured from one step (the same kernels, without the host's "
                         "per-launch work between them), the eager mean reported beside it; "
                         "0: from eager launches")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="before the steps, copy MIB MiB device to device once (a kernel "
                         "of known traffic that calibrates the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    w = synth.WORKLOADS[args.workload]
    if args.seg_len > 0:
        w = w.with_(seg_len=args.seg_len)
    rule = args.rule or w.rules[-1]
    pool, procs = None, 0
    if args.mode == "forward" and not args.no_cpu_baseline:
        procs = max(1, min(args.cpu_procs, os.cpu_count() or 1))
        pool = cpu_pool(procs)  # before the GPU is touched

    import torch

    import compressive_memory_transformers_amd as lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "decode":
        print(json.dumps(bench_decode(lib, w, rule, dev, args)), flush=True)
        return
    if args.mode == "backward":
        print(json.dumps(bench_backward(lib, w, rule, dev, args)), flush=True)
        return
    if args.mode == "block":
        print(json.dumps(bench_block(lib, w, rule, dev, args)), flush=True)
        return
    inp = synth.make_inputs(w, dev)
    out = torch.empty((w.B, w.Hq, w.L, w.d_value), dtype=inp["q"].dtype, device=dev)
    M = torch.empty_like(inp["M0"])
    z = torch.empty_like(inp["z0"])
    full, _ = lib.workspace_size_kv(w.B, w.Hq, w.Hkv, w.L, w.d, w.d_value, w.seg_len, rule,
                                    inp["q"].dtype)
    ws = torch.empty(full if args.plan == "overlapped" else full - 1, dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"],
                    w.seg_len, rule, out=out, M_final=M, z_final=z, workspace=ws,
                    stream=stream, events=events)

    if args.copy_probe > 0:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-phase events for every timed step; recorded once first so each
    # underlying HIP event exists before the library records it
    phase = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for evs in phase:
        for e in evs:
            e.record(stream)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        step(phase[k])
    end.record(stream)
    torch.cuda.synchronize()

    ms = start.elapsed_time(end) / args.steps
    scan_ms = sum(e[0].elapsed_time(e[1]) for e in phase) / args.steps
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in phase) / args.steps
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in phase)
    median_ms = step_ms[len(step_ms) // 2]

    # the same step captured once into a HIP graph and replayed: the same
    # kernels on the same buffers, without the host's per-launch work
    # between them
    graph_ms, graph_error = None, None
    if args.graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                lib.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["M0"], inp["z0"],
                            w.seg_len, rule, out=out, M_final=M, z_final=z, workspace=ws,
                            stream=torch.cuda.current_stream(dev))
        except RuntimeError as e:  # capture refused: the eager timing stands
            g, graph_error = None, str(e)[:200]
            torch.cuda.synchronize()
        if g is not None:
            for _ in range(args.warmup):
                g.replay()
            gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            gs.record(stream)
            for _ in range(args.steps):
                g.replay()
            ge.record(stream)
            torch.cuda.synchronize()
            graph_ms = gs.elapsed_time(ge) / args.steps
            del g
    eager_ms = ms
    if graph_ms is not None:
        ms = graph_ms

    # cold: each step after a 512 MiB device copy (outside its events) that
    # evicts the inputs from L2 and the 256 MB MALL
    cold_ms = None
    if args.cold > 0:
        a_ = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        b_ = torch.empty_like(a_)
        cold = []
        for _ in range(args.cold):
            b_.copy_(a_)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            for e in evs:
                e.record(stream)
            step(evs)
            torch.cuda.synchronize()
            cold.append(evs[0].elapsed_time(evs[2]))
        cold_ms = sorted(cold)[len(cold) // 2]
        del a_, b_

    # the shader clock, sampled while steps keep the GPU busy
    sclk = []
    for _ in range(args.sclk_samples):
        for _ in range(max(8, int(200 / max(ms, 1e-3)))):
            step()
        v_ = gpu_sclk_mhz()
        if v_ is not None:
            sclk.append(v_)
        torch.cuda.synchronize()
    sclk_mhz = sorted(sclk)[len(sclk) // 2] if sclk else None

    tokens = w.B * w.L
    flops = synth.flops(w, rule)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    if uses_fused_plan(w):
        # one kernel does the whole forward: its work is the call's
        a_flops = synth.flops(w, rule)
        a_bytes = synth.hbm_bytes(w)
        kname = "fused_kernel (the whole forward in one pass, state on chip)"
    else:
        a_flops = attn_kernel_flops(w)
        a_bytes = attn_kernel_bytes(w)
        kname = ("attn_kernel (local causal attention + retrieval + gate)" if w.d_value == w.d
                 else f"attn_kernel, d_key {w.d} != d_value {w.d_value} (attention + retrieval + "
                      "gate)")
    a_tflops = a_flops / (attn_ms * 1e-3) / 1e12
    traffic = measured_traffic(w, rule)
    # the bound is the kernel's: matrix cores above the ridge point
    # (peak FLOP/s / peak bytes/s), HBM below it
    if a_flops / a_bytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        roofline = {"kernel": kname,
                    "bound": "mfma", "achieved": a_tflops, "peak": peak, "unit": "TFLOP/s",
                    "frac": a_tflops / peak}
    else:
        gbs = a_bytes / (attn_ms * 1e-3) / 1e9
        roofline = {"kernel": kname,
                    "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": gbs / PEAK_HBM_GBS}
    roofline.update({"traffic": traffic, "algorithmic_flop_per_launch": a_flops,
                     "algorithmic_bytes_per_launch": a_bytes})
    rec = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian Q/K/V in HBM; random beta; M0 = 0, z0 = 1e-6)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "L": w.L, "d": w.d,
                   "seg_len": w.seg_len, "segments": w.segments, "rule": rule,
                   **({"d_value": w.d_value} if w.d_value != w.d else {})},
        "tflops": tflops,
        "frac_of_peak": tflops / peak,
        "peak_tflops": peak,
        "head_tokens_per_s": w.B * w.Hq * w.L / (ms * 1e-3),
        "hbm_gbs_compulsory": synth.hbm_bytes(w) / (ms * 1e-3) / 1e9,
        "phase_ms": {"scan_exposed": scan_ms, "attn": attn_ms},
        "plan": args.plan,
        "timing": ("replays of a HIP graph captured from one step" if graph_ms is not None
                   else "eager launches"),
        "eager_ms_per_step": eager_ms,
        "graph_error": graph_error,
        "ms_per_step_median": median_ms,
        "cold_ms_per_step_median": cold_ms,
        "sclk_mhz": sclk_mhz,
        "frac_of_clock_adjusted_peak": (tflops / (peak * sclk_mhz / 2400.0)
                                        if sclk_mhz else None),
        "roofline": roofline,
        "cpu_baseline": None,
        "pages_context": PAGES_CONTEXT,
    }
    if pool is not None:
        del inp
        rec["cpu_baseline"] = cpu_baseline(pool, procs, w, rule, args.cpu_seconds)
        pool.close()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
