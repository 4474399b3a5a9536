"""KV footprint closed forms (oracle).

* INMS walkthrough, sec. 1.2: n agents of average length L with a common prefix
  fraction p and per-token KV size s take n*L*s independently and about
  ((1 - p) * n + p) * L * s when the common part is stored once.  Its worked
  example (8 agents, p = 0.6, 16k tokens, 512 KiB per token) gives 64 GiB and,
  by the formula, 30.4 GiB (the page prints about 34 GB; the formula is used).
  Its three-agent example (8k tokens, 56 % common, 0.5 MB per token) gives 12 GB
  and 7.52 GB.
* INMS walkthrough, sec. 1.2: per token per layer a 7B MHA model with hidden
  size 4096 in fp16 stores 2 * 4096 * 2 bytes.
* Shared-memory prefix cache blog, sec. 1.1: per token, layers * 2 * kv_heads *
  head_dim * bytes (28 * 2 * 2 * 128 * 2 = 28672 B for its 7B GQA model).
"""
from __future__ import annotations


def independent(n: int, L: float, s: float) -> float:
    return n * L * s


def shared(n: int, L: float, s: float, p: float) -> float:
    return ((1.0 - p) * n + p) * L * s


def kv_bytes_per_token_mha(hidden: int, dtype_bytes: int, layers: int = 1) -> int:
    return 2 * hidden * dtype_bytes * layers


def kv_bytes_per_token_gqa(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return layers * 2 * kv_heads * head_dim * dtype_bytes


def shared_prefix_blocks(n: int, prefix_blocks: int, total_blocks: int) -> int:
    """Physical block count for n agents of total_blocks blocks that share the first
    prefix_blocks blocks: the closed form with p = prefix/total and L in blocks."""
    p = prefix_blocks / total_blocks
    return round(shared(n, total_blocks, 1, p))
