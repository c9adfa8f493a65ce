"""fp64 CPU oracle for the Infini-attention block forward and its gradients.

This package is TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it. The product
path (the HIP library and its Python binding) never imports it, and it imports
nothing from the product path: the two share no code. Its inputs are plain
numpy arrays; its arithmetic is numpy float64.

Sources (page title, then section):

* "Infini-Attention" (AI Wiki), section "What happens inside the
  Infini-attention block?": the local causal softmax attention A_dot, the
  memory retrieval A_mem = sigma(Q) M / (sigma(Q) z) with sigma = ELU + 1, and
  the per-head sigmoid gate A = sigmoid(beta) A_mem + (1 - sigmoid(beta)) A_dot.
* same page, section "How does the compressive memory work?": the delta-rule
  update of M, the update of z, and the additive (linear) variant.
* same page, section "Why is the memory footprint bounded?": segments of fixed
  length N, with the state (M, z) carried and nothing else.
* same page, section "What happens inside the Infini-attention block?" again:
  the input projections (query, key, value) and the output projection after
  the gate (oracle/block.py).
* same page, section "How is an Infini-attention model trained?": gradients
  flow through the memory recurrence as in truncated backpropagation through
  time (the backward pass; one call is the truncation window).
* "Hugging Face Infini-Attention Reproduction Analysis", section
  "Infini-Attention Mechanism", steps 1-6: the per-segment order (segment,
  local attention, retrieval from M_{s-1}, gate, update, carry only the
  memory).

Pins (each function is checked against something other than itself in
``tests/test_oracle_pins.py``):

* ``feature_map``       -- torch ``elu`` + 1, special values.
* ``gate_weight``       -- ``scipy.special.expit``.
* ``local_causal_attention`` -- torch ``scaled_dot_product_attention``
  (fp64, is_causal) and a per-token scalar softmax loop.
* ``memory_retrieval``  -- the block-strictly-causal quadratic form (closed
  form of the linear recurrence), causal linear attention at seg_len 1,
  constant-value invariant, a hand-worked example in exact dyadic rationals.
* ``memory_update`` (linear) -- segmentation independence and the one-shot
  sums over all keys, the hand-worked example.
* ``memory_update`` (delta)  -- the hand-worked two-segment d = 2 example,
  zero-residual invariance, the d = 1 scalar closed form, equality with the
  linear rule from a zero memory, joint linearity in (V, M0), the affine
  transition form.
* ``forward``           -- single-segment reduction to causal attention,
  gate extremes, chunked calls with a carried state, GQA equal to MHA on
  repeated K/V, batch/head permutation.
* ``forward_rows``, ``attend_last_row`` -- equal to ``forward`` (and to the
  last row of ``local_causal_attention``) on every row of small streams,
  both rules, grouped heads, ragged segments; the state equals ``forward``'s
  (``tests/test_oracle_rows.py``).
* ``decode_step``       -- token-by-token decoding of a stream equals
  ``forward`` on it (every output row, and the state at every segment end);
  the first token of a segment attends to itself alone (closed form); the
  state is unchanged inside a segment.
* ``block_forward``, ``project_qkv``, ``project_out`` (oracle/block.py) --
  scaled-permutation weights give an element-by-element closed form (each
  projected value is one input feature times a constant, read by explicit
  index arithmetic); linearity of y in the output weight; homogeneity in the
  value weights; four planted mistakes in the head split or the
  concatenation fail those checks (``tests/test_oracle_block.py``).
* ``backward`` (oracle/gradients.py) -- every gradient (Q, K, V, beta, M0,
  z0) against central finite differences of ``forward``, both rules, ragged,
  grouped and one-token segments; five planted mistakes (a dropped carry, a
  dropped term, a wrong derivative) fail that check
  (``tests/test_oracle_backward.py``).

No function here is "parity unpinned".
"""

from .infini_attention import (  # noqa: F401
    RULES,
    feature_map,
    gate_weight,
    local_causal_attention,
    memory_retrieval,
    memory_update,
    num_segments,
    forward,
    forward_rows,
    attend_last_row,
    decode_step,
)
from .gradients import backward  # noqa: F401
from .block import block_forward, project_out, project_qkv  # noqa: F401
from .compare import max_rel_err, slice_errors  # noqa: F401
