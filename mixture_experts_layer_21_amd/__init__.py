"""MI355X (gfx950) forward of a top-k token-choice MoE layer.

The compute lives in ``libmoe.so`` (hand-written HIP kernels behind a C ABI,
declared in include/moe.h); this package is its thin Python binding.
Importing it fails loudly when the library has not been built.
"""
from ._binding import (  # noqa: F401
    EXPORTED, LIB_PATH, MoeConfig, MoeError, backward_workspace_bytes, capacity, check_config,
    make_config, max_rows, moe_backward, moe_combine, moe_forward, moe_forward_noalloc,
    moe_grouped_swiglu,
    moe_permute, moe_rmsnorm, moe_route, moe_update_bias, new_saved, new_workspace,
    saved_bytes, status_string, workspace_bytes,
)
