"""Dense per-agent materialisation and decode attention (oracle, float64).

Sharing is a storage change only: each agent's attention must come out exactly
as if its whole context were stored densely (INMS walkthrough, sec. 1.3: dedup,
not compression, no information lost; TokenDance write-up, evaluation: the
master/mirror path adds no error of its own).  So the oracle builds every
agent's dense K and V and runs the plain attention of the MemDecay blog, sec.
4.2: scores q.k / sqrt(head_dim), softmax, weighted sum of V.  Grouped-query
attention: q head h reads kv head floor(h * Hkv / Hq) (contiguous groups; the
pages do not fix this).  The query attends to every cached token of its agent
(the current token is already cached), so no causal mask is needed.  An agent
with no cached tokens gets a zero output (a convention; the pages do not cover
it).

Two ways of materialising the dense context are given, and a test checks they
agree bit for bit:

* ``dense_plain``: straight from the workload's logical description -- what
  agent j reads at logical block b is its delta if it has one, else the block's
  content; K is moved from the content's storage frame to the block's position
  by the RoPE offset compensation (``oracle.rope``), the delta first, then the
  rotation (TokenDance write-up, sec. 3: correct the block, then restore RoPE).
* ``dense_from_tables``: through the oracle's own dedup tables and a pool that
  stores each physical block once.
"""
from __future__ import annotations

import numpy as np

from workload import rng as _rng
from workload import spec as _spec

from . import q4 as _q4
from . import rope as _rope


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """q [Hq, d]; K, V [L, Hkv, d] -> out [Hq, d], all float64."""
    q = np.asarray(q, np.float64)
    Hq, d = q.shape
    L, Hkv, _ = K.shape
    out = np.zeros((Hq, d), np.float64)
    if L == 0:
        return out
    grp = Hq // Hkv
    for h in range(Hq):
        g = h // grp
        s = (K[:, g, :] @ q[h]) * scale
        m = s.max()
        p = np.exp(s - m)
        out[h] = (p @ V[:, g, :]) / p.sum()
    return out


class _Store:
    """Stored block contents (float64) of one layer, generated on demand and memoised."""

    def __init__(self, wl, layer: int):
        self.wl, self.layer, self.memo = wl, layer, {}

    def get(self, seed16: bytes, ntok: int, g: int):
        key = (seed16, g)
        v = self.memo.get(key)
        if v is None:
            sh = self.wl.shape
            kb = _spec.block_kv_bits(seed16, sh, self.layer, ntok, _rng.SEL_K, head=g)[:ntok]
            vb = _spec.block_kv_bits(seed16, sh, self.layer, ntok, _rng.SEL_V, head=g)[:ntok]
            if sh.kv_dtype == _spec.Q4G64:
                kc, kp = _rng.q4_encode(kb)
                vc, vp = _rng.q4_encode(vb)
                k = _q4.dequant(kc, kp)
                v_ = _q4.dequant(vc, vp)
            else:
                k = _rng.bf16_bits_to_f32(kb).astype(np.float64)
                v_ = _rng.bf16_bits_to_f32(vb).astype(np.float64)
            v = (k, v_)
            self.memo[key] = v
        return v


def _kv_heads(wl, heads):
    sh = wl.shape
    grp = sh.n_q_heads // sh.n_kv_heads
    if heads is None:
        return list(range(sh.n_kv_heads))
    return sorted({h // grp for h in heads})


def _assemble(wl, store, j, kvh, blocks):
    """blocks: list of (seed16, ntok, shift).  Returns K, V [L, Hkv, d] (unused
    kv heads left zero)."""
    sh = wl.shape
    L = sum(nt for _, nt, _ in blocks)
    K = np.zeros((L, sh.n_kv_heads, sh.head_dim), np.float64)
    V = np.zeros_like(K)
    t = 0
    for seed16, nt, shift in blocks:
        for g in kvh:
            k, v = store.get(seed16, nt, g)
            K[t:t + nt, g] = _rope.rotate(k, shift, sh.rope_theta) if shift else k
            V[t:t + nt, g] = v
        t += nt
    return K, V


def dense_plain(wl, j: int, store, kvh):
    blocks = []
    for b in range(wl.n_blocks(j)):
        shift = int(wl.blk_pos0[j][b]) - int(wl.blk_frame[j][b])
        blocks.append((_spec.logical_seed(wl, j, b), int(wl.blk_ntok[j][b]), shift))
    return _assemble(wl, store, j, kvh, blocks)


def _phys_seed(wl, tables, p: int) -> bytes:
    j, b = int(tables["phys_agent"][p]), int(tables["phys_block"][p])
    if p >= tables["n_dedup"]:
        return wl.blk_delta_seed[j][b]
    return wl.blk_seed[j][b]


def dense_from_tables(wl, tables, j: int, store, kvh):
    blocks = []
    for b in range(int(tables["n_blocks"][j])):
        e = int(tables["delta_table"][j, b])
        if e < 0:
            e = int(tables["block_table"][j, b])
        blocks.append((_phys_seed(wl, tables, e), int(tables["phys_ntok"][e]), int(tables["shift"][j, b])))
    return _assemble(wl, store, j, kvh, blocks)


def decode(wl, layer: int = 0, agents=None, heads=None, tables=None, q=None) -> np.ndarray:
    """Decode-step attention of every (or the given) agent for one layer.

    Returns float64 [n_agents_selected, Hq, d]; q heads not in ``heads`` are 0.
    With ``tables`` the dense context is rebuilt through them, else from the
    logical description.  ``q`` (bf16 bits [n, Hq, d]) defaults to the
    workload's seeded queries for the layer.
    """
    sh = wl.shape
    if q is None:
        q = _spec.q_bits(wl, layer)
    qf = _rng.bf16_bits_to_f32(q).astype(np.float64)
    agents = list(range(wl.n_agents)) if agents is None else list(agents)
    hsel = list(range(sh.n_q_heads)) if heads is None else list(heads)
    kvh = _kv_heads(wl, hsel)
    store = _Store(wl, layer)
    scale = 1.0 / np.sqrt(sh.head_dim)
    out = np.zeros((len(agents), sh.n_q_heads, sh.head_dim), np.float64)
    for i, j in enumerate(agents):
        if tables is None:
            K, V = dense_plain(wl, j, store, kvh)
        else:
            K, V = dense_from_tables(wl, tables, j, store, kvh)
        o = attend(qf[j], K, V, scale)
        out[i, hsel] = o[hsel]
    return out
