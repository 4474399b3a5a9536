"""Master/mirror diff construction and restore (oracle).

TokenDance write-up, sec. 3: the round keeps one dense master cache and stores
every other cache as a mirror -- a reference to the master plus block-sparse
K/V differences; restoring a mirror applies its differences and puts the keys
back at the mirror's positions (RoPE) on the way into paged memory.

* ``diff_flags``: does a mirror's candidate block differ from its master block?
  Only valid token slots count.  Threshold 0: any bit differs; threshold t > 0:
  some |candidate - master| > t, or a NaN on either side.  The threshold test
  decides an integer, so it is taken in float32 (the difference of two bf16
  values rounded once to float32, t rounded to float32), as the device takes it.
* ``restore_blocks``: agent j's blocks as a restore writes them: per logical
  block, the delta block if the agent has one there, else the table's block;
  valid tokens' K moved by R(shift) and rounded to bf16 (nearest even), V as
  stored, padding slots zero.

Readings taken: differences are decided per whole block (every layer, kv head,
K and V), matching the block-granular deltas; candidates are given in the
master's stored frame, the frame deltas are kept in.
"""
from __future__ import annotations

import numpy as np

from . import rope as _rope
from .lifecycle import bf16_round


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def diff_flags(master_k, master_v, cand_k, cand_v, ntok, tau: float) -> np.ndarray:
    """master_* / cand_*: uint16 bf16 bits [n, L, Hkv, B, d]; ntok [n].
    Returns int32 [n]: 1 where the candidate differs, else 0."""
    n = len(ntok)
    out = np.zeros(n, np.int32)
    for i in range(n):
        nt = int(ntok[i])
        for a, b in ((master_k[i], cand_k[i]), (master_v[i], cand_v[i])):
            a, b = a[:, :, :nt], b[:, :, :nt]
            if tau == 0:
                d = np.any(a != b)
            else:
                fa = bf16_bits_to_f64(a).astype(np.float32)
                fb = bf16_bits_to_f64(b).astype(np.float32)
                d = np.any(~(np.abs(fa - fb) <= np.float32(tau)))
            if d:
                out[i] = 1
    return out


def restore_blocks(tables: dict, j: int, stored, B: int, base: float):
    """stored(p) -> (K, V) float64 [ntok, Hkv, d] stored-frame contents of
    physical block p (bf16 values).  Returns float64 K, V [m, B, Hkv, d] as the
    restore writes agent j's m logical blocks (padding slots zero)."""
    m = int(tables["n_blocks"][j])
    Ks, Vs = [], []
    for b in range(m):
        e = int(tables["delta_table"][j, b])
        if e < 0:
            e = int(tables["block_table"][j, b])
        nt = int(tables["ntok"][j, b])
        shift = int(tables["shift"][j, b])
        K, V = stored(e)
        K, V = np.asarray(K, np.float64)[:nt], np.asarray(V, np.float64)[:nt]
        if shift:
            K = bf16_round(_rope.rotate(K, shift, base))
        k = np.zeros((B,) + K.shape[1:])
        v = np.zeros_like(k)
        k[:nt], v[:nt] = K, V
        Ks.append(k)
        Vs.append(v)
    return np.array(Ks), np.array(Vs)
