"""DDTree tree-verify hot path for AMD Instinct MI355X (gfx950).

The work happens in ``libddtree.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/ddtree.h``); ``_lib`` is a thin ctypes binding
with the same entry-point names, and ``step`` chains the four stages on
device tensors.
"""
from ._lib import (  # noqa: F401
    DDTREE_BF16,
    DDTREE_F32,
    DDTreeError,
    ddtree_abi_version,
    ddtree_accept,
    ddtree_build_tree,
    ddtree_compile_visibility,
    ddtree_verify_attn,
    ddtree_verify_attn_workspace_size,
    load,
)
