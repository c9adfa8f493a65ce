"""The Infini-attention block forward, written out plainly in numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring). Slow on purpose: one
(batch, KV-head) unit at a time, one segment at a time, the full score matrix
of each segment materialised and masked.

Readings taken where the pages leave a step open:

* softmax scale 1/sqrt(d_key): the block page writes sqrt(d_model) but also
  says the local path is standard attention, which scales by the per-head key
  width;
* one (M, z) per (batch element, KV head) with M of shape (d_key, d_value);
  query heads that share a KV head (grouped-query attention) read the same
  memory, and kv_head = q_head // (Hq // Hkv);
* ELU with alpha = 1, so sigma(x) = x + 1 for x > 0 and exp(x) otherwise;
* the denominators sigma(q) . z are one scalar per row, broadcast over d_value,
  with no extra epsilon;
* retrieval and the delta-rule prediction both use the state from before the
  segment (M_{s-1}, z_{s-1}); the delta rule is a batched update over the whole
  segment, not a token-by-token one;
* the causal mask keeps the diagonal (key u is visible to query t iff u <= t)
  and never crosses a segment boundary;
* a final segment shorter than seg_len when L is not a multiple of it;
* sigma is applied to the unscaled Q and K; 1/sqrt(d) appears only inside the
  softmax;
* beta has one value per query head, shared across the batch, and
  sigmoid(beta) multiplies A_mem.
"""

import math

import numpy as np

RULES = ("linear", "delta")


def feature_map(x):
    """sigma(x) = ELU(x) + 1 with alpha = 1, elementwise.

    "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
    block?": the linear-attention feature map applied to queries (retrieval)
    and keys (update).
    """
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def gate_weight(beta):
    """sigmoid(beta): the weight of A_mem in the per-head gate.

    "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
    block?", equation for A.
    """
    beta = float(beta)
    if beta >= 0.0:
        return 1.0 / (1.0 + math.exp(-beta))
    e = math.exp(beta)
    return e / (1.0 + e)


def local_causal_attention(q, k, v):
    """A_dot for one head and one segment: causal softmax(q k^T / sqrt(d)) v.

    q: [n, d_key], k: [n, d_key], v: [n, d_value]; row t attends to rows
    u <= t of the same segment only.

    "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
    block?", equation for A_dot; "Hugging Face Infini-Attention Reproduction
    Analysis", "Infini-Attention Mechanism", step 2.
    """
    n, d_key = q.shape
    scores = (q @ k.T) / math.sqrt(d_key)
    future = np.triu(np.ones((n, n), dtype=bool), k=1)
    scores = np.where(future, -np.inf, scores)
    scores = scores - scores.max(axis=1, keepdims=True)
    weights = np.exp(scores)
    return (weights @ v) / weights.sum(axis=1, keepdims=True)


def memory_retrieval(q, M, z):
    """A_mem = sigma(q) M / (sigma(q) z), one scalar denominator per row.

    q: [n, d_key], M: [d_key, d_value], z: [d_key].

    "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
    block?", equation for A_mem; "Hugging Face Infini-Attention Reproduction
    Analysis", "Infini-Attention Mechanism", step 3.
    """
    sq = feature_map(q)
    return (sq @ M) / (sq @ z)[:, None]


def memory_update(k, v, M, z, rule):
    """One segment's update of (M, z); returns the new pair.

    linear: M_s = M_{s-1} + sigma(K)^T V
    delta:  M_s = M_{s-1} + sigma(K)^T (V - sigma(K) M_{s-1} / (sigma(K) z_{s-1}))
    both:   z_s = z_{s-1} + sum_t sigma(K_t)

    k: [n, d_key], v: [n, d_value], M: [d_key, d_value], z: [d_key].

    "Infini-Attention" (AI Wiki), "How does the compressive memory work?":
    the delta rule, the z update, and the additive variant.
    """
    if rule not in RULES:
        raise ValueError(f"unknown update rule {rule!r}")
    sk = feature_map(k)
    if rule == "linear":
        M_new = M + sk.T @ v
    else:
        predicted = (sk @ M) / (sk @ z)[:, None]
        M_new = M + sk.T @ (v - predicted)
    z_new = z + sk.sum(axis=0)
    return M_new, z_new


def num_segments(L, seg_len):
    """Number of segments of a length-L stream: ceil(L / seg_len)."""
    return -(-L // seg_len)


def forward(q, k, v, beta, M0, z0, seg_len, rule, units=None, out_segments=None):
    """The block forward over all segments.

    q: [B, Hq, L, d_key]; k: [B, Hkv, L, d_key]; v: [B, Hkv, L, d_value];
    beta: [Hq]; M0: [B, Hkv, d_key, d_value]; z0: [B, Hkv, d_key].
    Returns (out [B, Hq, L, d_value], M_final, z_final) as float64.

    ``units``: optional list of (b, kv_head) pairs to compute; the outputs of
    every other unit are NaN. ``out_segments``: optional set of segment indices
    whose output rows are computed; the state chain still runs over every
    segment (the state never depends on the local path), and the other output
    rows are NaN. Neither option changes the arithmetic of what is computed.

    Per segment, in the order of "Hugging Face Infini-Attention Reproduction
    Analysis", "Infini-Attention Mechanism", steps 1-6: local attention,
    retrieval from the previous memory, the gate, then the update; only
    (M, z) is carried to the next segment ("Infini-Attention" (AI Wiki), "Why
    is the memory footprint bounded?").
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    M0 = np.asarray(M0, dtype=np.float64)
    z0 = np.asarray(z0, dtype=np.float64)
    B, Hq, L, _ = q.shape
    Hkv = k.shape[1]
    d_value = v.shape[3]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if seg_len < 1:
        raise ValueError("seg_len must be >= 1")
    group = Hq // Hkv
    S = num_segments(L, seg_len)
    if units is None:
        units = [(b, j) for b in range(B) for j in range(Hkv)]

    out = np.full((B, Hq, L, d_value), np.nan)
    M_final = np.full(M0.shape, np.nan)
    z_final = np.full(z0.shape, np.nan)
    for b, j in units:
        M = M0[b, j].copy()
        z = z0[b, j].copy()
        for s in range(S):
            t0, t1 = s * seg_len, min((s + 1) * seg_len, L)
            k_s, v_s = k[b, j, t0:t1], v[b, j, t0:t1]
            if out_segments is None or s in out_segments:
                for h in range(j * group, (j + 1) * group):
                    q_s = q[b, h, t0:t1]
                    a_dot = local_causal_attention(q_s, k_s, v_s)
                    a_mem = memory_retrieval(q_s, M, z)
                    g = gate_weight(beta[h])
                    out[b, h, t0:t1] = g * a_mem + (1.0 - g) * a_dot
            M, z = memory_update(k_s, v_s, M, z, rule)
        M_final[b, j] = M
        z_final[b, j] = z
    return out, M_final, z_final



def attend_last_row(q_t, k_prefix, v_prefix):
    """A_dot of one query row: softmax(q_t k^T / sqrt(d)) v over the rows of
    its segment up to and including its own (k_prefix, v_prefix: [t + 1, d]).

    The last row of ``local_causal_attention`` on the same block, computed
    alone in O(t d): what the causal mask leaves of the segment is exactly
    this prefix ("Infini-Attention" (AI Wiki), "What happens inside the
    Infini-attention block?", equation for A_dot).
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    k_prefix = np.asarray(k_prefix, dtype=np.float64)
    v_prefix = np.asarray(v_prefix, dtype=np.float64)
    scores = (k_prefix @ q_t) / math.sqrt(q_t.shape[0])
    weights = np.exp(scores - scores.max())
    return (weights @ v_prefix) / weights.sum()


def forward_rows(q, k, v, beta, M0, z0, seg_len, rule, rows):
    """``forward`` restricted to the output rows ``rows`` (token indices, the
    same for every batch element and head), for segments too long for the
    N x N score matrix.

    Returns (out_rows [B, Hq, len(rows), d_value], M_final, z_final). The
    state chain runs over every segment as in ``forward``; each requested row
    t of segment s is the gate of attend_last_row over the segment's rows up
    to t and of the retrieval of q_t from the state before s.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, Hq, L, _ = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    S = num_segments(L, seg_len)
    rows = [int(t) for t in rows]
    if any(t < 0 or t >= L for t in rows):
        raise ValueError("rows must lie in [0, L)")
    by_seg = {}
    for r, t in enumerate(rows):
        by_seg.setdefault(t // seg_len, []).append((r, t))
    out = np.full((B, Hq, len(rows), v.shape[3]), np.nan)
    M_final = np.full(np.shape(M0), np.nan)
    z_final = np.full(np.shape(z0), np.nan)
    for b in range(B):
        for j in range(Hkv):
            M = np.asarray(M0, dtype=np.float64)[b, j].copy()
            z = np.asarray(z0, dtype=np.float64)[b, j].copy()
            for s in range(S):
                t0, t1 = s * seg_len, min((s + 1) * seg_len, L)
                for r, t in by_seg.get(s, []):
                    for h in range(j * group, (j + 1) * group):
                        q_t = q[b, h, t]
                        a_dot = attend_last_row(q_t, k[b, j, t0:t + 1], v[b, j, t0:t + 1])
                        a_mem = memory_retrieval(q_t[None, :], M, z)[0]
                        g = gate_weight(beta[h])
                        out[b, h, r] = g * a_mem + (1.0 - g) * a_dot
                M, z = memory_update(k[b, j, t0:t1], v[b, j, t0:t1], M, z, rule)
            M_final[b, j] = M
            z_final[b, j] = z
    return out, M_final, z_final

def decode_step(q, k, v, beta, M, z, k_cache, v_cache, pos, seg_len, rule):
    """One streaming step: the token at position ``pos`` (0-based) of its segment.

    q: [B, Hq, d_key]; k: [B, Hkv, d_key]; v: [B, Hkv, d_value] for the new
    token. M: [B, Hkv, d_key, d_value], z: [B, Hkv, d_key]: the state before
    the token's segment. k_cache / v_cache: [B, Hkv, seg_len, d]: rows
    0 .. pos-1 hold the segment's earlier tokens. Returns
    (out [B, Hq, d_value], M', z', k_cache', v_cache'), all float64 copies.

    The token's key and value join the cache at row ``pos``; its query attends
    causally to rows 0 .. pos of the segment, reads the memory of the previous
    segments, and the two are gated, exactly as row ``pos`` of the segment in
    ``forward``. When the segment is full (pos == seg_len - 1) it is folded
    into (M, z) with ``memory_update`` and M', z' are the state after it;
    otherwise M', z' equal M, z.

    "Infini-Attention" (AI Wiki), "Why is the memory footprint bounded?": a
    stream is processed segment by segment with only (M, z) carried, so the
    work per token does not grow with the stream; "What happens inside the
    Infini-attention block?" for the per-token arithmetic.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    M = np.array(M, dtype=np.float64)
    z = np.array(z, dtype=np.float64)
    k_cache = np.array(k_cache, dtype=np.float64)
    v_cache = np.array(v_cache, dtype=np.float64)
    B, Hq, d_key = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if not 0 <= pos < seg_len or k_cache.shape[2] != seg_len:
        raise ValueError("pos must lie in [0, seg_len) and the cache hold seg_len rows")
    group = Hq // Hkv
    out = np.empty((B, Hq, v.shape[2]))
    for b in range(B):
        for j in range(Hkv):
            k_cache[b, j, pos] = k[b, j]
            v_cache[b, j, pos] = v[b, j]
            keys, values = k_cache[b, j, :pos + 1], v_cache[b, j, :pos + 1]
            for h in range(j * group, (j + 1) * group):
                scores = keys @ q[b, h] / math.sqrt(d_key)
                weights = np.exp(scores - scores.max())
                a_dot = weights @ values / weights.sum()
                a_mem = memory_retrieval(q[b, h][None, :], M[b, j], z[b, j])[0]
                g = gate_weight(beta[h])
                out[b, h] = g * a_mem + (1.0 - g) * a_dot
            if pos == seg_len - 1:
                M[b, j], z[b, j] = memory_update(k_cache[b, j], v_cache[b, j], M[b, j], z[b, j],
                                                 rule)
    return out, M, z, k_cache, v_cache
