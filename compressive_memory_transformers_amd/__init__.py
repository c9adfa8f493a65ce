"""Infini-attention block on AMD Instinct MI355X (gfx950): forward, decode step, backward,
and the block with its input and output projections.

The computation lives in libinfini_attn.so (hand-written HIP kernels behind
the C ABI of include/infini_attn.h); this package is its thin Python binding.
Importing it loads the library and fails loudly if it is not built.
"""

from .binding import (  # noqa: F401
    DTYPES,
    RULES,
    InfiniAttnError,
    backward,
    backward_workspace_size,
    block_forward,
    block_workspace_size,
    decode_step,
    decode_workspace_size,
    forward,
    forward_noalloc,
    forward_train,
    load_library,
    status_string,
    version,
    workspace_size,
    workspace_size_kv,
)

load_library()
