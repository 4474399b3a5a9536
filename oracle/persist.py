"""Persistent Q4 block pool (oracle) -- test infrastructure.

Q4 KV paper summary, sec. 2.1: each agent's cache is cut into fixed blocks kept
in Q4 form in safetensors files, one namespace per agent; sec. 2.2: a cache is
loaded back while another agent decodes.

* ``q4_image``: the bytes an agent's blocks occupy in a saved image -- for each
  of K codes, V codes, K params, V params (in that order) the listed blocks of
  every layer, layer-major: tensor[layer][ids[i]] for i in order.
* ``scatter``: the pool after an image is loaded into blocks ids.

Readings: a block is saved with every layer of the pool and both K and V (the
unit the pages persist is the agent's whole cache); the file also carries each
block's valid-token count; the format is checked against the safetensors
library itself (the page names the format, not a layout of our own).
"""
from __future__ import annotations

import numpy as np


def q4_image(k_codes, v_codes, k_params, v_params, ids) -> bytes:
    """Pools as numpy arrays [L][P][...] (codes uint8, params float16)."""
    ids = list(ids)
    parts = []
    for t in (k_codes, v_codes, k_params, v_params):
        sel = np.stack([t[:, i] for i in ids], 1) if ids else t[:, :0]
        parts.append(np.ascontiguousarray(sel).tobytes())
    return b"".join(parts)


def scatter(pools, image: bytes, ids):
    """pools: list of four numpy arrays [L][P][...] (copied, not modified);
    returns them with image block i written to pool block ids[i]."""
    out = [p.copy() for p in pools]
    n = len(ids)
    off = 0
    for t in out:
        L = t.shape[0]
        blk = t[0, 0].nbytes
        size = L * n * blk
        part = np.frombuffer(image[off:off + size], dtype=t.dtype).reshape((L, n) + t.shape[2:])
        for i, p in enumerate(ids):
            t[:, p] = part[:, i]
        off += size
    return out
