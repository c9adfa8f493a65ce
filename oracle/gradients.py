"""Gradients of the Infini-attention block forward, numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring). Slow on purpose: one
(batch, KV-head) unit at a time, one segment at a time, every score matrix
materialised.

"Infini-Attention" (AI Wiki), "How is an Infini-attention model trained?":
during training, gradients flow through the memory recurrence from segment
to segment, as in truncated backpropagation through time. Reading taken: one
call of the block is the truncation window. Gradients flow back through every
segment of the call, through both the local path and the memory, down to the
initial state (M0, z0), whose gradients are returned; nothing flows past it.

The function differentiates exactly what ``infini_attention.forward``
computes: a scalar loss is taken to be
    sum(d_out * out) + sum(dM_final * M_final) + sum(dz_final * z_final),
and the gradients of that loss with respect to every input are returned. Each
helper below is the chain rule applied to one step of the forward, in the
reverse of the forward's order; the finite-difference pins in the tests check
every term.
"""

import math

import numpy as np

from .infini_attention import RULES, feature_map, gate_weight, num_segments


def feature_map_grad(x):
    """d sigma / dx for sigma(x) = ELU(x) + 1: 1 above zero, e^x at or below.

    Both sides give 1 at x = 0, so the derivative is continuous there.
    """
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))


def update_backward(k_s, v_s, M_prev, z_prev, dM, dz, rule):
    """Backward of one segment's memory update.

    Forward ("Infini-Attention" (AI Wiki), "How does the compressive memory
    work?"): with Phi = sigma(K_s),
      linear: M_s = M_prev + Phi^T V_s
      delta:  M_s = M_prev + Phi^T (V_s - P / c), P = Phi M_prev, c = Phi z_prev
      both:   z_s = z_prev + sum_t Phi_t
    Given dM = dL/dM_s and dz = dL/dz_s, returns (dk_s, dv_s, dM_prev, dz_prev):
    the update's contributions to dL/dK_s and dL/dV_s, and dL/dM_prev,
    dL/dz_prev through the update (the retrieval adds its own later).
    """
    phi = feature_map(k_s)
    dphi = np.broadcast_to(dz, phi.shape).copy()  # z_s = z_prev + sum_t phi_t
    dM_prev = dM.copy()
    dz_prev = dz.copy()
    if rule == "linear":
        dv_s = phi @ dM                 # M_s[i, j] += phi_t[i] v_t[j]
        dphi += v_s @ dM.T
    elif rule == "delta":
        c = phi @ z_prev                # one scalar per row
        pred = (phi @ M_prev) / c[:, None]
        u = v_s - pred
        du = phi @ dM                   # M_s = M_prev + Phi^T U
        dphi += u @ dM.T
        dv_s = du.copy()                # U = V - pred
        dpred = -du
        dp = dpred / c[:, None]         # pred = P / c
        dc = -(dpred * pred).sum(axis=1) / c
        dphi += dp @ M_prev.T           # P = Phi M_prev
        dM_prev += phi.T @ dp
        dphi += dc[:, None] * z_prev[None, :]  # c = Phi z_prev
        dz_prev += phi.T @ dc
    else:
        raise ValueError(f"unknown update rule {rule!r}")
    dk_s = dphi * feature_map_grad(k_s)
    return dk_s, dv_s, dM_prev, dz_prev


def retrieval_backward(q_s, M_prev, z_prev, da_mem):
    """Backward of A_mem = sigma(Q) M_prev / (sigma(Q) z_prev).

    "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
    block?", equation for A_mem. Given da_mem = dL/dA_mem, returns
    (dq_s, dM_prev, dz_prev) contributions.
    """
    sq = feature_map(q_s)
    num = sq @ M_prev
    den = sq @ z_prev
    a_mem = num / den[:, None]
    dnum = da_mem / den[:, None]
    dden = -(da_mem * a_mem).sum(axis=1) / den
    dsq = dnum @ M_prev.T + dden[:, None] * z_prev[None, :]
    return dsq * feature_map_grad(q_s), sq.T @ dnum, sq.T @ dden


def local_attention_backward(q_s, k_s, v_s, da_dot):
    """Backward of A_dot = causal softmax(Q K^T / sqrt(d)) V for one head.

    "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
    block?", equation for A_dot. Returns (dq_s, dk_s, dv_s).
    """
    n, d_key = q_s.shape
    scale = 1.0 / math.sqrt(d_key)
    scores = (q_s @ k_s.T) * scale
    future = np.triu(np.ones((n, n), dtype=bool), k=1)
    scores = np.where(future, -np.inf, scores)
    p = np.exp(scores - scores.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    dv_s = p.T @ da_dot
    dp = da_dot @ v_s.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))  # softmax rows
    return (ds @ k_s) * scale, (ds.T @ q_s) * scale, dv_s


def local_attention(q_s, k_s, v_s):
    """A_dot for one head (as infini_attention.local_causal_attention)."""
    n, d_key = q_s.shape
    scores = (q_s @ k_s.T) / math.sqrt(d_key)
    future = np.triu(np.ones((n, n), dtype=bool), k=1)
    scores = np.where(future, -np.inf, scores)
    p = np.exp(scores - scores.max(axis=1, keepdims=True))
    return (p @ v_s) / p.sum(axis=1, keepdims=True)


def backward(q, k, v, beta, M0, z0, seg_len, rule, d_out, dM_final=None, dz_final=None,
             units=None):
    """Gradients of the block forward over all segments of one call.

    Shapes as ``infini_attention.forward``; d_out like out, dM_final like M0,
    dz_final like z0 (None: zero). Returns (dq, dk, dv, dbeta, dM0, dz0) as
    float64. ``units``: optional list of (b, kv_head) pairs; the gradients of
    every other unit's rows and state are NaN, and dbeta sums over the listed
    units only.

    Per unit: the forward is run once to record the state before each segment;
    then the segments are walked in reverse. In segment s the incoming dM, dz
    are the gradients with respect to the state after s. The update step is
    undone first (it was the segment's last step), then, for every query head
    of the group, the gate, the retrieval (which read M_{s-1}, z_{s-1}) and
    the local attention. What reaches M_{s-1}, z_{s-1} is carried to segment
    s - 1.
    """
    if rule not in RULES:
        raise ValueError(f"unknown update rule {rule!r}")
    f64 = lambda x: np.asarray(x, dtype=np.float64)
    q, k, v, beta, M0, z0, d_out = map(f64, (q, k, v, beta, M0, z0, d_out))
    B, Hq, L, _ = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    S = num_segments(L, seg_len)
    dM_final = np.zeros(M0.shape) if dM_final is None else f64(dM_final)
    dz_final = np.zeros(z0.shape) if dz_final is None else f64(dz_final)
    if units is None:
        units = [(b, j) for b in range(B) for j in range(Hkv)]

    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    dbeta = np.zeros(Hq)
    dM0 = np.full(M0.shape, np.nan)
    dz0 = np.full(z0.shape, np.nan)
    for b, j in units:
        states = []
        M, z = M0[b, j].copy(), z0[b, j].copy()
        for s in range(S):
            t0, t1 = s * seg_len, min((s + 1) * seg_len, L)
            states.append((M.copy(), z.copy()))
            M, z = _update(k[b, j, t0:t1], v[b, j, t0:t1], M, z, rule)
        dM, dz = dM_final[b, j].copy(), dz_final[b, j].copy()
        for s in reversed(range(S)):
            t0, t1 = s * seg_len, min((s + 1) * seg_len, L)
            k_s, v_s = k[b, j, t0:t1], v[b, j, t0:t1]
            M_prev, z_prev = states[s]
            dk_s, dv_s, dM, dz = update_backward(k_s, v_s, M_prev, z_prev, dM, dz, rule)
            for h in range(j * group, (j + 1) * group):
                q_s, do = q[b, h, t0:t1], d_out[b, h, t0:t1]
                g = gate_weight(beta[h])
                sq = feature_map(q_s)
                a_mem = (sq @ M_prev) / (sq @ z_prev)[:, None]
                a_dot = local_attention(q_s, k_s, v_s)
                # out = g A_mem + (1 - g) A_dot, g = sigmoid(beta_h)
                dbeta[h] += (do * (a_mem - a_dot)).sum() * g * (1.0 - g)
                dq_m, dM_r, dz_r = retrieval_backward(q_s, M_prev, z_prev, g * do)
                dq_a, dk_a, dv_a = local_attention_backward(q_s, k_s, v_s, (1.0 - g) * do)
                dq[b, h, t0:t1] = dq_m + dq_a
                dk_s = dk_s + dk_a
                dv_s = dv_s + dv_a
                dM = dM + dM_r
                dz = dz + dz_r
            dk[b, j, t0:t1] = dk_s
            dv[b, j, t0:t1] = dv_s
        dM0[b, j] = dM
        dz0[b, j] = dz
    return dq, dk, dv, dbeta, dM0, dz0


def _update(k_s, v_s, M, z, rule):
    # the forward's update, imported late so a test may replace it
    from .infini_attention import memory_update
    return memory_update(k_s, v_s, M, z, rule)
