"""Deduplicated paged KV pool and decode attention for MI355X (gfx950).

The compute path lives in ``libkvpool.so`` (C ABI in ``include/kvpool.h``);
this package is its thin ctypes binding (``_lib``) and the in-tree build
(``build``).
"""
from ._lib import (DevicePlan, KvpError, Tables, build_tables, kv_rerotate,  # noqa: F401
                   paged_decode_attn, workspace_bytes)
