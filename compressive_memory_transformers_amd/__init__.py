"""Infini-attention block forward on AMD Instinct MI355X (gfx950).

The computation lives in libinfini_attn.so (hand-written HIP kernels behind
the C ABI of include/infini_attn.h); this package is its thin Python binding.
Importing it loads the library and fails loudly if it is not built.
"""

from .binding import (  # noqa: F401
    DTYPES,
    RULES,
    InfiniAttnError,
    decode_step,
    decode_workspace_size,
    forward,
    load_library,
    status_string,
    version,
    workspace_size,
)

load_library()
