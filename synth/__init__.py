"""Seeded synthetic inputs for the Infini-attention block forward.

This module holds the workload table and the input generators, and nothing of
the method's arithmetic. Both sides of every parity check (the HIP library and
the fp64 oracle) receive the same tensors made here; the oracle reads them back
as float64 on the host.

Every (tensor, batch, head) slice is drawn from its own torch generator, seeded
from ``numpy.random.SeedSequence([config_seed, tensor_id, b, h])``, so any slice
can be regenerated alone. Draws are N(0, 1) in float32, scaled in float32 where
a workload asks for it, then rounded to the workload's dtype (round to nearest
even for bfloat16). The same seed gives different numbers on a CPU and on a GPU
generator; a parity check always gives both sides one set of tensors.

The pages evaluate on PG19, Arxiv-math, BookSum and passkey data; none of that
is used. These Gaussian inputs take the shapes the pages describe instead:
2048-token segments and a 1M-token stream ("Infini-Attention" (AI Wiki),
"Why is the memory footprint bounded?" and "Can Infini-attention retrieve a
passkey at one million tokens?"), and 16 rollouts of 64-token segments
("Hugging Face Infini-Attention Reproduction Analysis", "Weight Decay and
Rollouts").
"""

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "beta": 3, "outlier": 4, "x": 5, "w_qkv": 6,
              "w_o": 7, "M0": 8}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    seg_len: int
    dtype: str  # "f32" or "bf16"
    rules: tuple
    seed: int
    key_std: float = 1.0
    key_outlier_p: float = 0.0
    key_outlier_scale: float = 1.0
    z0: float = 1e-6
    dv: int = 0  # the value width when it differs from the key width d
    note: str = field(default="", compare=False)

    @property
    def d_value(self):
        return self.dv or self.d

    @property
    def segments(self):
        return -(-self.L // self.seg_len)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload(
        "tiny", B=1, Hq=2, Hkv=2, L=64, d=32, seg_len=16, dtype="f32",
        rules=("linear",), seed=0,
        note="B1 H2 d32, 4 segments of 16, fp32, linear rule"),
    "hf_repro": Workload(
        "hf_repro", B=8, Hq=16, Hkv=16, L=1024, d=64, seg_len=64, dtype="bf16",
        rules=("linear", "delta"), seed=1,
        note="B8 H16 d64, 16 rollouts of 64-token segments, bf16"),
    "llama3_8b": Workload(
        "llama3_8b", B=4, Hq=32, Hkv=8, L=32768, d=128, seg_len=2048,
        dtype="bf16", rules=("delta",), seed=2,
        note="B4, 32 query / 8 KV heads, d128, 16 segments of 2048, bf16"),
    "long_stream": Workload(
        "long_stream", B=1, Hq=16, Hkv=16, L=1048576, d=128, seg_len=2048,
        dtype="bf16", rules=("linear",), seed=3, key_std=1.0 / math.sqrt(128),
        note="B1 H16 d128, 512 segments of 2048 (1M tokens), keys std 1/sqrt(d)"),
    "small_segment": Workload(
        "small_segment", B=16, Hq=32, Hkv=32, L=32768, d=128, seg_len=128,
        dtype="bf16", rules=("delta",), seed=4, key_outlier_p=0.05,
        key_outlier_scale=8.0,
        note="B16 H32 d128, 256 segments of 128, 5% of key rows scaled by 8"),
    "long_segment": Workload(
        "long_segment", B=1, Hq=16, Hkv=16, L=400000, d=128, seg_len=100000,
        dtype="bf16", rules=("linear",), seed=5, key_std=1.0 / math.sqrt(128),
        note="B1 H16 d128, 4 segments of 100000 tokens (very long segments)"),
    "kv_split": Workload(
        "kv_split", B=4, Hq=32, Hkv=8, L=32768, d=64, dv=128, seg_len=2048,
        dtype="bf16", rules=("delta",), seed=6,
        note="the llama3_8b layer with 64-wide keys and 128-wide values (d_key != d_value)"),
}


def slice_seed(config_seed, tensor, b, h):
    """64-bit seed of one (tensor, batch, head) slice."""
    ss = np.random.SeedSequence([config_seed, TENSOR_IDS[tensor], b, h])
    return int(ss.generate_state(1, dtype=np.uint64)[0])


def _normal(shape, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _uniform(shape, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def make_inputs(w, device="cpu"):
    """Inputs of workload ``w`` on ``device``.

    Returns a dict with q [B,Hq,L,d], k [B,Hkv,L,d] and v [B,Hkv,L,dv] in the
    workload's dtype, beta [Hq] float32, M0 [B,Hkv,d,dv] float32 (zeros) and
    z0 [B,Hkv,d] float32 (all ``w.z0``); dv is ``w.d_value``.
    """
    dt = w.torch_dtype
    dv = w.d_value
    q = torch.empty((w.B, w.Hq, w.L, w.d), dtype=dt, device=device)
    k = torch.empty((w.B, w.Hkv, w.L, w.d), dtype=dt, device=device)
    v = torch.empty((w.B, w.Hkv, w.L, dv), dtype=dt, device=device)
    for b in range(w.B):
        for h in range(w.Hq):
            q[b, h] = _normal((w.L, w.d), slice_seed(w.seed, "q", b, h), device).to(dt)
        for h in range(w.Hkv):
            kk = _normal((w.L, w.d), slice_seed(w.seed, "k", b, h), device)
            if w.key_std != 1.0:
                kk = kk * w.key_std
            if w.key_outlier_p > 0.0:
                pick = _uniform((w.L,), slice_seed(w.seed, "outlier", b, h), device)
                kk = torch.where((pick < w.key_outlier_p)[:, None],
                                 kk * w.key_outlier_scale, kk)
            k[b, h] = kk.to(dt)
            v[b, h] = _normal((w.L, dv), slice_seed(w.seed, "v", b, h), device).to(dt)
    beta = _normal((w.Hq,), slice_seed(w.seed, "beta", 0, 0), device)
    M0 = torch.zeros((w.B, w.Hkv, w.d, dv), dtype=torch.float32, device=device)
    z0 = torch.full((w.B, w.Hkv, w.d), w.z0, dtype=torch.float32, device=device)
    return dict(q=q, k=k, v=v, beta=beta, M0=M0, z0=z0)


def make_unit_inputs(w, b, j):
    """The slices of one (batch b, KV head j) unit of workload ``w``, drawn
    on the CPU from the same per-slice seeds as ``make_inputs`` and rounded to
    the workload's dtype, as float64 numpy arrays with leading dimensions of
    size 1: q [1, G, L, d] (the G = Hq / Hkv query heads of KV head j), k
    [1, 1, L, d], v [1, 1, L, dv], beta [G], M0 [1, 1, d, dv], z0 [1, 1, d]."""
    dt = w.torch_dtype
    dv = w.d_value
    G = w.Hq // w.Hkv
    q = torch.empty((1, G, w.L, w.d), dtype=dt)
    for g in range(G):
        q[0, g] = _normal((w.L, w.d), slice_seed(w.seed, "q", b, j * G + g), "cpu").to(dt)
    kk = _normal((w.L, w.d), slice_seed(w.seed, "k", b, j), "cpu")
    if w.key_std != 1.0:
        kk = kk * w.key_std
    if w.key_outlier_p > 0.0:
        pick = _uniform((w.L,), slice_seed(w.seed, "outlier", b, j), "cpu")
        kk = torch.where((pick < w.key_outlier_p)[:, None], kk * w.key_outlier_scale, kk)
    k = kk.to(dt)[None, None]
    v = _normal((w.L, dv), slice_seed(w.seed, "v", b, j), "cpu").to(dt)[None, None]
    beta = _normal((w.Hq,), slice_seed(w.seed, "beta", 0, 0), "cpu")[j * G:(j + 1) * G]
    M0 = torch.zeros((1, 1, w.d, dv), dtype=torch.float32)
    z0 = torch.full((1, 1, w.d), w.z0, dtype=torch.float32)
    return {n: to_f64(t) for n, t in dict(q=q, k=k, v=v, beta=beta, M0=M0, z0=z0).items()}


def to_f64(t):
    """A tensor (any dtype, any device) as a float64 numpy array on the host."""
    return t.detach().to("cpu", torch.float32).double().numpy()


def flops(w, rule):
    """Algorithmic matrix-product FLOPs of one forward call.

    Per (query head, token): 2d(N+1) for the causal QK^T and PV with the
    diagonal counted (the mean of 2d per visible key over a segment of N is
    2d(N+1)/2 each for QK^T and PV), 2d^2 for sigma(Q) M, and per (KV head,
    token) 2d^2 (linear) or 4d^2 (delta) for the update. Summed exactly over
    segments so a short final segment is counted as it is. With a value width
    dv: (d + dv)(N+1) for the two local products and d dv in place of d^2.
    """
    d, dv = w.d, w.d_value
    per_seg = []
    for s in range(w.segments):
        n = min(w.seg_len, w.L - s * w.seg_len)
        local = (d + dv) * n * (n + 1)  # both products over the causal triangle
        retrieval = 2 * n * d * dv
        update = (2 if rule == "linear" else 4) * n * d * dv
        per_seg.append(w.Hq * (local + retrieval) + w.Hkv * update)
    return w.B * sum(per_seg)


def hbm_bytes(w):
    """Compulsory HBM bytes of one call: Q, K, V read once, out written once,
    the fp32 state read and written once, beta read once."""
    e = 4 if w.dtype == "f32" else 2
    d, dv = w.d, w.d_value
    return (e * w.L * w.B * ((d + dv) * w.Hq + (d + dv) * w.Hkv)
            + 8 * w.B * w.Hkv * (d * dv + d) + 4 * w.Hq)


def make_block_inputs(B, L, d_model, Hq, Hkv, d, dtype, device="cpu", seed=0, z0=1e-6,
                      m0_scale=0.0, dv=None):
    """Inputs of the block with its projections, on ``device``.

    x [B, L, d_model] N(0, 1); w_qkv [(Hq + Hkv) d + Hkv dv, d_model] (query
    and key heads d rows each, value heads dv rows; dv = d unless given) and
    w_o [d_model, Hq dv], each N(0, 1 / fan_in) (random weights: the projected
    values then have unit variance), in ``dtype``; beta [Hq] N(0, 1) float32;
    M0 [B, Hkv, d, dv] float32, N(0, m0_scale^2) (zeros by default); z0
    [B, Hkv, d] float32, all ``z0``. Slices are seeded per batch element (x)
    and per head (the weights' row blocks).
    """
    dv = d if dv is None else dv
    x = torch.empty((B, L, d_model), dtype=dtype, device=device)
    for b in range(B):
        x[b] = _normal((L, d_model), slice_seed(seed, "x", b, 0), device).to(dtype)
    widths = [d] * (Hq + Hkv) + [dv] * Hkv
    w_qkv = torch.empty((sum(widths), d_model), dtype=dtype, device=device)
    r0 = 0
    for h, wd in enumerate(widths):
        w_qkv[r0:r0 + wd] = (_normal((wd, d_model), slice_seed(seed, "w_qkv", 0, h), device)
                             / math.sqrt(d_model)).to(dtype)
        r0 += wd
    w_o = (_normal((d_model, Hq * dv), slice_seed(seed, "w_o", 0, 0), device)
           / math.sqrt(Hq * dv)).to(dtype)
    beta = _normal((Hq,), slice_seed(seed, "beta", 0, 0), device)
    M0 = torch.zeros((B, Hkv, d, dv), dtype=torch.float32, device=device)
    if m0_scale:
        for b in range(B):
            for h in range(Hkv):
                M0[b, h] = m0_scale * _normal((d, dv), slice_seed(seed, "M0", b, h), device)
    z0 = torch.full((B, Hkv, d), z0, dtype=torch.float32, device=device)
    return dict(x=x, w_qkv=w_qkv, w_o=w_o, beta=beta, M0=M0, z0=z0)


def block_flops(B, L, d_model, Hq, Hkv, d, seg_len, rule):
    """Algorithmic FLOPs of the block with its projections: the input
    projection 2 B L d_model (Hq + 2 Hkv) d, the block forward (``flops``),
    the output projection 2 B L Hq d d_model."""
    w = Workload("block", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, seg_len=seg_len, dtype="bf16",
                 rules=(rule,), seed=0)
    proj = 2 * B * L * d_model * (Hq + 2 * Hkv) * d + 2 * B * L * Hq * d * d_model
    return proj + flops(w, rule)
