"""RoPE offset compensation (oracle).

INMS walkthrough, sec. 2.3 and sec. 3.2: a stored key carries the rotation of
its original position; when the block is reused at another position the key is
rotated once more by an angle that depends only on the position difference
(target minus source); values are not touched.

Reading taken (the pages fix no pairing or base): rotate-half pairing of
element i with element i + d/2, frequency theta_i = base**(-2 i / d), and
R(delta) rotates each pair by +delta * theta_i, so a key at position a moved to
b = a + delta is R(delta) k.  All arithmetic in float64.
"""
from __future__ import annotations

import numpy as np


def inv_freq(head_dim: int, base: float) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * i / head_dim)


def rotate(x: np.ndarray, delta, base: float) -> np.ndarray:
    """R(delta) x over the last axis.  ``delta`` broadcasts against x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(delta, dtype=np.float64)[..., None] * inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
