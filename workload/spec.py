"""Seeded synthetic multi-agent workloads (spans, tokens, deltas, content seeds).

These stand in for the pages' workloads, whose traces and models are not
available: INMS-style agents sharing a global prefix (INMS walkthrough, sec. 1.2
and sec. 4.1), TokenDance all-gather rounds in which every agent's prompt holds
the previous round's outputs as shared segments behind a private history of
varying length (TokenDance write-up, "memory pain" and sec. 1-3), and the
persistent Q4 cache's private 256-token blocks (Q4 KV paper summary, sec. 2.1).

What this module decides, and nothing more:

* the span structure of every agent (tier, group, kind, tokens);
* which logical blocks of mirrors carry a delta (block-sparse K/V difference);
* a 16-byte *content seed* per logical block, from which K/V values are drawn
  (``workload.rng``).  Two logical blocks get the same seed exactly when they
  hold the same cached content: same sharing domain (tier, group, and for
  private spans the owning agent and span), same chain root kind, and the same
  token history from that root through the end of the block.  A PREFIX span
  continues the chain of the block before it; a SEGMENT span restarts it, so a
  segment's content does not depend on where it is placed.
* ``frame_pos``: the logical start position of the first logical block (agents
  in order, blocks in order) with the same seed.  Stored K is post-RoPE in that
  frame.  A delta block is stored in its master block's frame.

Tokens are uniform in [1, 2**30); 0 is never emitted (a reserved separator).
"""
from __future__ import annotations

import hashlib
import struct
from dataclasses import dataclass, field

import numpy as np

from . import rng as _rng

# Tier / kind / dtype codes (same numbering as the C ABI).
GLOBAL, GROUP, PRIVATE = 0, 1, 2
PREFIX, SEGMENT = 0, 1
BF16, Q4G64 = 0, 1


@dataclass
class Shape:
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_tokens: int
    kv_dtype: int = BF16
    rope_theta: float = 10000.0


@dataclass
class Span:
    tier: int
    group: int
    kind: int
    tokens: np.ndarray  # int32


@dataclass
class Agent:
    spans: list
    delta_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))


@dataclass
class Workload:
    name: str
    seed: int
    shape: Shape
    agents: list
    # per agent, per logical block descriptors (filled by describe())
    blk_span: list = None      # span index
    blk_tok0: list = None      # first token index within the span
    blk_ntok: list = None
    blk_pos0: list = None      # logical start position (dst_pos0)
    blk_seed: list = None      # list of 16-byte seeds
    blk_frame: list = None     # frame_pos of the content
    blk_delta_seed: list = None  # dict b -> 16-byte seed

    @property
    def n_agents(self):
        return len(self.agents)

    def n_blocks(self, j):
        return len(self.blk_ntok[j])

    def context_len(self, j):
        return int(sum(len(s.tokens) for s in self.agents[j].spans))


# ----------------------------------------------------------------------------
# content seeds


def _h(*parts: bytes) -> bytes:
    m = hashlib.blake2b(digest_size=16)
    for p in parts:
        m.update(p)
    return m.digest()


ROOT_AGENT = _h(b"root:agent-start")
ROOT_SEGMENT = _h(b"root:segment-start")


def _domain(span: Span, j: int, si: int) -> bytes:
    if span.tier == PRIVATE:
        return struct.pack("<iiii", PRIVATE, 0, j, si)
    if span.tier == GROUP:
        return struct.pack("<iiii", GROUP, span.group, -1, -1)
    return struct.pack("<iiii", GLOBAL, 0, -1, -1)


def delta_seed(wl_seed: int, name: str, j: int, b: int) -> bytes:
    return _h(b"delta", name.encode(), struct.pack("<qii", wl_seed, j, b))


def describe(wl: Workload) -> Workload:
    """Cut every span into blocks and attach the per-block descriptors."""
    B = wl.shape.block_tokens
    wl.blk_span, wl.blk_tok0, wl.blk_ntok, wl.blk_pos0 = [], [], [], []
    wl.blk_seed, wl.blk_frame, wl.blk_delta_seed = [], [], []
    first_pos = {}
    for j, ag in enumerate(wl.agents):
        bs, bt, bn, bp, bseed, bfr = [], [], [], [], [], []
        pos = 0
        prev = ROOT_AGENT
        for si, sp in enumerate(ag.spans):
            n = len(sp.tokens)
            if sp.kind == SEGMENT:
                prev = ROOT_SEGMENT
            dom = _domain(sp, j, si)
            for t0 in range(0, n, B):
                t1 = min(n, t0 + B)
                seed = _h(prev, dom, np.ascontiguousarray(sp.tokens[t0:t1], dtype="<i4").tobytes())
                prev = seed
                bs.append(si)
                bt.append(t0)
                bn.append(t1 - t0)
                bp.append(pos + t0)
                bseed.append(seed)
                if seed not in first_pos:
                    first_pos[seed] = pos + t0
                bfr.append(first_pos[seed])
            pos += n
        wl.blk_span.append(np.array(bs, np.int32))
        wl.blk_tok0.append(np.array(bt, np.int32))
        wl.blk_ntok.append(np.array(bn, np.int32))
        wl.blk_pos0.append(np.array(bp, np.int32))
        wl.blk_seed.append(bseed)
        wl.blk_frame.append(np.array(bfr, np.int64))
        wl.blk_delta_seed.append({int(b): delta_seed(wl.seed, wl.name, j, int(b)) for b in ag.delta_blocks})
    return wl


def segment_block_ids(wl: Workload, j: int) -> np.ndarray:
    """Logical block indices of agent j that belong to SEGMENT spans of a shared tier."""
    sp = wl.agents[j].spans
    return np.array([b for b, si in enumerate(wl.blk_span[j])
                     if sp[si].kind == SEGMENT and sp[si].tier != PRIVATE], np.int32)


# ----------------------------------------------------------------------------
# generators


def _rs(seed: int, cfg: int, purpose: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, purpose]))


def _tokens(g: np.random.Generator, n: int) -> np.ndarray:
    return g.integers(1, 1 << 30, size=n, dtype=np.int64).astype(np.int32)


def _delta_runs(g: np.random.Generator, seg_ranges, m: int) -> np.ndarray:
    """Pick m block indices clustered at segment boundaries.

    Visit segments in a seeded order and take a run of 1-3 blocks from each
    segment's first block; if budget remains, runs ending at each segment's last
    block; then grow the runs inward one block at a time until m are chosen.
    """
    chosen = set()
    order = g.permutation(len(seg_ranges))
    lead = {}   # segment -> next inward index from the front
    trail = {}  # segment -> next inward index from the back
    budget = m
    for s in order:
        if budget <= 0:
            break
        a, b = seg_ranges[s]
        r = min(int(g.integers(1, 4)), b - a, budget)
        for x in range(a, a + r):
            chosen.add(x)
        lead[s] = a + r
        budget = m - len(chosen)
    if budget > 0:
        for s in order:
            if budget <= 0:
                break
            a, b = seg_ranges[s]
            r = min(int(g.integers(1, 4)), budget)
            x = b - 1
            k = 0
            while k < r and x >= lead.get(s, a):
                if x not in chosen:
                    chosen.add(x)
                    k += 1
                x -= 1
            trail[s] = x
            budget = m - len(chosen)
    while len(chosen) < m:
        grew = False
        for s in order:
            if len(chosen) >= m:
                break
            a, b = seg_ranges[s]
            x = lead.get(s, a)
            if x < b and x not in chosen:
                chosen.add(x)
                lead[s] = x + 1
                grew = True
            elif x < b:
                lead[s] = x + 1
                grew = True
            if len(chosen) >= m:
                break
            y = trail.get(s, b - 1)
            if y >= a and y not in chosen:
                chosen.add(y)
                trail[s] = y - 1
                grew = True
            elif y >= a:
                trail[s] = y - 1
                grew = True
        if not grew:
            break
    return np.array(sorted(chosen), np.int32)


def tiny(seed: int = 0) -> Workload:
    """C1: 4 agents, GQA 4/2, d 64, B 16; global prefix 128 + private tails U{32..96}."""
    g = _rs(seed, 1, 0)
    prefix = _tokens(g, 128)
    agents = []
    for j in range(4):
        t = int(g.integers(32, 97))
        agents.append(Agent([Span(GLOBAL, 0, PREFIX, prefix), Span(PRIVATE, 0, PREFIX, _tokens(g, t))]))
    return describe(Workload("tiny", seed, Shape(1, 4, 2, 64, 16, BF16, 10000.0), agents))


def inms(seed: int = 0, n_agents: int = 8, ctx: int = 16384, prefix_len: int = 9824) -> Workload:
    """C2: 8 agents, MHA 32x128, B 16, 16384 tokens with a 9824-token global prefix."""
    g = _rs(seed, 2, 0)
    prefix = _tokens(g, prefix_len)
    agents = [Agent([Span(GLOBAL, 0, PREFIX, prefix), Span(PRIVATE, 0, PREFIX, _tokens(g, ctx - prefix_len))])
              for _ in range(n_agents)]
    return describe(Workload("inms", seed, Shape(1, 32, 32, 128, 16, BF16, 10000.0), agents))


def _round(seed, cfg, name, n_agents, shape, priv_rng, seg_rng, frac_fn, seg_count=None):
    g = _rs(seed, cfg, 0)
    n_seg = n_agents if seg_count is None else seg_count
    priv_len = g.integers(priv_rng[0], priv_rng[1] + 1, size=n_agents)
    seg_len = g.integers(seg_rng[0], seg_rng[1] + 1, size=n_seg)
    tg = _rs(seed, cfg, 1)
    segs = [_tokens(tg, int(n)) for n in seg_len]
    agents = []
    for j in range(n_agents):
        spans = [Span(PRIVATE, 0, PREFIX, _tokens(tg, int(priv_len[j])))]
        spans += [Span(GROUP, 0, SEGMENT, s) for s in segs]
        agents.append(Agent(spans))
    wl = Workload(name, seed, shape, agents)
    dg = _rs(seed, cfg, 2)
    B = shape.block_tokens
    for j in range(1, n_agents):
        f = frac_fn(dg)
        # segment ranges in this agent's logical block numbering
        nb_priv = -(-int(priv_len[j]) // B)
        ranges, b = [], nb_priv
        for n in seg_len:
            nb = -(-int(n) // B)
            ranges.append((b, b + nb))
            b += nb
        n_segblocks = b - nb_priv
        m = int(round(f * n_segblocks))
        agents[j].delta_blocks = _delta_runs(dg, ranges, m)
    return describe(wl)


def tokendance(seed: int = 0) -> Workload:
    """C3: 64 agents, 40/8 heads, d 128, theta 1e6, B 16; private U{512..4096} +
    64 group segments U{128..512} in the same order; mirrors carry deltas on
    U(0.03, 0.09) of their segment blocks."""
    return _round(seed, 3, "tokendance", 64, Shape(1, 40, 8, 128, 16, BF16, 1e6),
                  (512, 4096), (128, 512), lambda g: float(g.uniform(0.03, 0.09)))


def q4(seed: int = 0) -> Workload:
    """C4: 12 private agents, 8192 tokens, B 256, GQA 32/8, d 128, Q4 groupwise."""
    g = _rs(seed, 4, 0)
    agents = [Agent([Span(PRIVATE, 0, PREFIX, _tokens(g, 8192))]) for _ in range(12)]
    return describe(Workload("q4", seed, Shape(1, 32, 8, 128, 256, Q4G64, 10000.0), agents))


def scale(seed: int = 0, n_layers: int = 48) -> Workload:
    """C5: 250 agents, 48 layers, 40/8 heads, d 128, theta 1e6, B 16; private
    U{1024..4096} + 250 group segments U{64..256}; mirrors 5 % delta blocks."""
    return _round(seed, 5, "scale", 250, Shape(n_layers, 40, 8, 128, 16, BF16, 1e6),
                  (1024, 4096), (64, 256), lambda g: 0.05)


# ---- small variants used by the parity tests ---------------------------------


def tiny_seg(seed: int = 0) -> Workload:
    """Three shared segments placed in a different order in every agent (so every
    agent has its own shift per segment), after private histories of different
    lengths; mirrors carry deltas; partial blocks everywhere."""
    g = _rs(seed, 11, 0)
    segs = [_tokens(g, int(n)) for n in g.integers(20, 51, size=3)]
    agents = []
    for j in range(4):
        order = g.permutation(3)
        spans = [Span(PRIVATE, 0, PREFIX, _tokens(g, int(g.integers(20, 61))))]
        spans += [Span(GROUP, 7, SEGMENT, segs[s]) for s in order]
        agents.append(Agent(spans))
    wl = describe(Workload("tiny_seg", seed, Shape(1, 4, 2, 64, 16, BF16, 10000.0), agents))
    for j in range(1, 4):
        sb = segment_block_ids(wl, j)
        k = int(g.integers(1, 3))
        agents[j].delta_blocks = np.sort(g.choice(sb, size=k, replace=False)).astype(np.int32)
    return describe(wl)


def tiny_q4(seed: int = 0, block_tokens: int = 16) -> Workload:
    """Global prefix + private tails with Q4 groupwise K/V, d 128 (two groups)."""
    g = _rs(seed, 12, 0)
    prefix = _tokens(g, 3 * block_tokens)
    agents = []
    for j in range(3):
        t = int(g.integers(block_tokens // 2, 3 * block_tokens))
        agents.append(Agent([Span(GLOBAL, 0, PREFIX, prefix), Span(PRIVATE, 0, PREFIX, _tokens(g, t))]))
    return describe(Workload("tiny_q4", seed, Shape(1, 4, 2, 128, block_tokens, Q4G64, 10000.0), agents))


def small_round(seed: int = 0, n_agents: int = 12, hq: int = 10, hkv: int = 2, block_tokens: int = 16) -> Workload:
    """A scaled-down TokenDance round (many rows per shared block, deltas, shifts)."""
    return _round(seed, 13, "small_round", n_agents, Shape(1, hq, hkv, 128, block_tokens, BF16, 1e6),
                  (40, 300), (20, 90), lambda g: float(g.uniform(0.03, 0.3)))


CONFIGS = {
    "tiny": tiny,
    "inms": inms,
    "tokendance": tokendance,
    "q4": q4,
    "scale": scale,
}


def make(name: str, seed: int = 0, **kw) -> Workload:
    fns = dict(CONFIGS)
    fns.update(tiny_seg=tiny_seg, tiny_q4=tiny_q4, small_round=small_round)
    return fns[name](seed, **kw)


# ----------------------------------------------------------------------------
# value draws


def q_bits(wl: Workload, layer: int) -> np.ndarray:
    """Decode queries for one layer: bf16 bits [n_agents, Hq, d]."""
    sh = wl.shape
    out = np.empty((wl.n_agents, sh.n_q_heads, sh.head_dim), np.uint16)
    for j in range(wl.n_agents):
        s = _rng.seed_words(_h(b"query", wl.name.encode(), struct.pack("<qi", wl.seed, j)))
        out[j] = _rng.bf16_tile(s, layer, _rng.SEL_Q, (sh.n_q_heads, sh.head_dim))
    return out


def block_kv_bits(seed16: bytes, shape: Shape, layer: int, ntok: int, sel: int, head=None) -> np.ndarray:
    """Stored K (sel=SEL_K) or V (SEL_V) of one block: bf16 bits [Hkv, B, d]
    (or [B, d] for one kv head); slots at and beyond ntok hold NaN (they must
    never be read)."""
    B, H, d = shape.block_tokens, shape.n_kv_heads, shape.head_dim
    sw = _rng.seed_words(seed16)
    if head is None:
        t = _rng.bf16_tile(sw, layer, sel, (H, B, d))
        t[:, ntok:, :] = _rng.BF16_NAN
    else:
        t = _rng.bf16_range(sw, layer, sel, head * B * d, B * d).reshape(B, d)
        t[ntok:, :] = _rng.BF16_NAN
    return t


def logical_seed(wl: Workload, j: int, b: int) -> bytes:
    """Seed of what agent j actually reads at logical block b (its delta if any)."""
    ds = wl.blk_delta_seed[j].get(b)
    return ds if ds is not None else wl.blk_seed[j][b]


def fingerprint(wl: Workload) -> str:
    """sha256 over everything that decides a workload's inputs: name, seed, shape
    and every agent's spans (tier, group, kind, tokens) and delta blocks.  Stored
    expected outputs carry it, so a changed generator shows up as a mismatch."""
    m = hashlib.sha256()
    sh = wl.shape
    m.update(wl.name.encode())
    m.update(struct.pack("<q7d", wl.seed, sh.n_layers, sh.n_q_heads, sh.n_kv_heads, sh.head_dim,
                         sh.block_tokens, sh.kv_dtype, sh.rope_theta))
    for ag in wl.agents:
        m.update(struct.pack("<i", len(ag.spans)))
        for sp in ag.spans:
            m.update(struct.pack("<iiii", sp.tier, sp.group, sp.kind, len(sp.tokens)))
            m.update(np.ascontiguousarray(sp.tokens, dtype="<i4").tobytes())
        d = np.ascontiguousarray(ag.delta_blocks, dtype="<i4")
        m.update(struct.pack("<i", len(d)))
        m.update(d.tobytes())
    return m.hexdigest()
