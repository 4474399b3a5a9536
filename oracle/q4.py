"""Groupwise 4-bit KV dequantisation (oracle).

Q4 KV paper summary, sec. 2.1-2.2: KV blocks are kept 4-bit quantised (a
compression of about 0.281 of fp16) and read by attention directly.  Format:
group of 64 consecutive head-dim elements, fp16 scale s and fp16 zero z per
group, code c in [0, 15] with the even element in the low nibble; the value is
x = s * c + z.  Computed in float64 (exact for these operands).
"""
from __future__ import annotations

import numpy as np

GROUP = 64


def dequant(codes: np.ndarray, params: np.ndarray) -> np.ndarray:
    """codes uint8 [..., d/2], params float16 [..., d/64, 2] -> float64 [..., d]."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = (codes & 0x0F).astype(np.float64)
    hi = (codes >> 4).astype(np.float64)
    c = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.float64)
    c[..., 0::2] = lo
    c[..., 1::2] = hi
    d = c.shape[-1]
    s = np.asarray(params[..., 0], dtype=np.float64)
    z = np.asarray(params[..., 1], dtype=np.float64)
    cg = c.reshape(*c.shape[:-1], d // GROUP, GROUP)
    return (s[..., None] * cg + z[..., None]).reshape(c.shape)


def compression_ratio(head_dim: int) -> float:
    """Bytes of the Q4 layout over bytes of fp16 for one head row."""
    q4 = head_dim // 2 + (head_dim // GROUP) * 4
    return q4 / (head_dim * 2)
