"""Paged single-token decode attention for MI355X (gfx950).

The compute path is the HIP library built from csrc/ (libpadecode.so); the
Python side only marshals torch tensors into its C ABI. Importing this package
does not load the library; `decode()` does, and raises if it is missing.
"""
from ._lib import (SPLIT_BALANCED, BlockPool, PaError, Prepared, decode, decode_noalloc, kv_append,
                   library_path, load_library, lse_merge, prefix_workspace_bytes, prepare,
                   reset_workspace, workspace_bytes)

__all__ = ["SPLIT_BALANCED", "BlockPool", "PaError", "Prepared", "decode", "decode_noalloc",
           "kv_append", "library_path", "load_library", "lse_merge", "prefix_workspace_bytes",
           "prepare", "reset_workspace", "workspace_bytes"]
