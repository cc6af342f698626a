"""RecSA (Recursive Sparse Attention) hot path for MI355X (gfx950).

The compute lives in librecsa.so (HIP kernels behind the C ABI in
include/recsa.h); `recsa` is the ctypes binding.
"""
from . import recsa  # noqa: F401
from .recsa import (  # noqa: F401
    Pooler, Tree, RecsaError, recsa_append_decode, recsa_attn_decode,
    recsa_attn_prefill, recsa_build_tree, recsa_decode, recsa_init_rope, recsa_level_rows,
    recsa_levels_needed, recsa_select, recsa_status_string,
    recsa_workspace_bytes, workspace,
)
