"""The projections around the block, numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
block?": for each segment the layer forms the usual query, key and value
projections of its input tokens, runs both attention paths on them, gates
the two results, and sends the gated result through the output matrix.

Readings taken where the page is silent:

* no biases;
* every weight is stored as a linear layer stores it, (out_features,
  in_features), and applied as x @ W^T;
* one fused input weight w_qkv of (Hq + 2 Hkv) d rows: the Hq query heads'
  rows first, then the Hkv key heads', then the Hkv value heads'; head h of a
  group takes the d consecutive rows h d .. h d + d - 1 of its group;
* the output projection reads the heads' gated results concatenated in head
  order along the feature axis (feature h d + j is element j of head h).

Shapes: x [B, L, d_model]; q [B, Hq, L, d], k and v [B, Hkv, L, d] (the
block's own layout); y [B, L, d_model].
"""

import numpy as np

from .infini_attention import forward


def project_qkv(x, w_qkv, Hq, Hkv, d):
    """q, k, v of the input tokens: one product with the fused weight, then
    the columns split into heads."""
    x = np.asarray(x, dtype=np.float64)
    w_qkv = np.asarray(w_qkv, dtype=np.float64)
    B, L, _ = x.shape
    assert w_qkv.shape[0] == (Hq + 2 * Hkv) * d
    y = x @ w_qkv.T                                   # [B, L, (Hq + 2 Hkv) d]

    def heads(cols, H):
        return y[..., cols].reshape(B, L, H, d).transpose(0, 2, 1, 3)

    q = heads(slice(0, Hq * d), Hq)
    k = heads(slice(Hq * d, (Hq + Hkv) * d), Hkv)
    v = heads(slice((Hq + Hkv) * d, (Hq + 2 * Hkv) * d), Hkv)
    return q, k, v


def project_out(a, w_o):
    """y = concat_h(a_h) @ w_o^T for a [B, Hq, L, d] (the gated result)."""
    a = np.asarray(a, dtype=np.float64)
    B, Hq, L, d = a.shape
    cat = a.transpose(0, 2, 1, 3).reshape(B, L, Hq * d)
    return cat @ np.asarray(w_o, dtype=np.float64).T


def block_forward(x, w_qkv, w_o, beta, M0, z0, seg_len, rule, Hq, Hkv, d):
    """The block with its projections: (y, M_final, z_final)."""
    q, k, v = project_qkv(x, w_qkv, Hq, Hkv, d)
    a, M, z = forward(q, k, v, beta, M0, z0, seg_len, rule)
    return project_out(a, w_o), M, z
