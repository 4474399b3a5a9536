"""Exact-key block dedup, refcounts and master/mirror delta tables (oracle).

Follows:
* INMS walkthrough, sec. 2.2: KV lives in fixed-size blocks; each block's
  content is fingerprinted and looked up in the pool of its tier; a hit reuses
  the physical block and increments its reference count, a miss allocates a new
  block; a sequence keeps hitting until its content forks.  Copy-on-write: when a
  sequence writes different content into a shared block it gets its own copy and
  the old block's count drops by one.
* INMS walkthrough, sec. 2.1 / 2.3 / 3.2: three tiers (global, group, private);
  only public blocks are shared, private blocks never; tier is part of the match.
* TokenDance write-up, sec. 1: segments are indexed by their own content, not by
  their absolute position, so a segment restarts the chain.
* TokenDance write-up, sec. 3: one dense master plus mirrors stored as
  block-sparse K/V differences (read here as whole replacement blocks).

Readings taken where the pages are silent:
* every span starts a new block; the last block of a span may be partial;
* a PREFIX block's key holds its predecessor's physical id (the chain); the
  first block of a SEGMENT span has the SEGMENT root as predecessor; a PRIVATE
  block's key also holds (agent, span index), so it is never shared;
* ids are given in first-occurrence order (agents in order, blocks in order);
  delta ids follow all dedup ids in (agent, block) order;
* refcount counts effective references: an entry overlaid by a delta does not
  count toward its master block (the copy-on-write decrement); a delta block
  has count 1;
* a delta block is stored in its master's frame: src_pos0(delta) =
  src_pos0(master); shift(j, b) = dst_pos0(j, b) - src_pos0(block_table[j][b]);
* deltas may be placed only on blocks of SEGMENT spans of a shared tier; the
  per-agent list must be strictly increasing and in range.

No hashing, no ordering tricks: a Python dict keyed by the full tuple.
"""
from __future__ import annotations

import numpy as np

GLOBAL, GROUP, PRIVATE = 0, 1, 2
PREFIX, SEGMENT = 0, 1

# status codes of the C ABI, used to compare error behaviour
EINVAL, ETIER = -1, -2

AGENT_ROOT = ("agent-root",)
SEG_ROOT = ("segment-root",)


class OracleError(ValueError):
    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


def build_tables(block_tokens: int, agents) -> dict:
    """agents: sequence of objects with ``spans`` (tier, group, kind, tokens) and
    ``delta_blocks``.  Returns a dict of numpy int32 arrays (see keys below)."""
    B = int(block_tokens)
    if B <= 0:
        raise OracleError(EINVAL, "block_tokens")
    ids = {}
    src_pos0, phys_ntok, phys_agent, phys_block = [], [], [], []
    per_agent = []  # list of lists of (id, ntok, dst_pos0, kind, tier)
    for j, ag in enumerate(agents):
        rows = []
        parent = AGENT_ROOT
        pos = 0
        for si, sp in enumerate(ag.spans):
            if sp.tier not in (GLOBAL, GROUP, PRIVATE) or sp.kind not in (PREFIX, SEGMENT):
                raise OracleError(EINVAL, "tier/kind")
            if sp.tier == GROUP and sp.group < 0:
                raise OracleError(ETIER, "group span without group id")
            toks = [int(t) for t in sp.tokens]
            if sp.kind == SEGMENT:
                parent = SEG_ROOT
            if sp.tier == PRIVATE:
                dom = (PRIVATE, 0, j, si)
            elif sp.tier == GROUP:
                dom = (GROUP, int(sp.group), -1, -1)
            else:
                dom = (GLOBAL, 0, -1, -1)
            for t0 in range(0, len(toks), B):
                chunk = tuple(toks[t0:t0 + B])
                key = (dom, parent, chunk)
                if key not in ids:
                    ids[key] = len(ids)
                    src_pos0.append(pos + t0)
                    phys_ntok.append(len(chunk))
                    phys_agent.append(j)
                    phys_block.append(len(rows))
                p = ids[key]
                rows.append((p, len(chunk), pos + t0, sp.kind, sp.tier))
                parent = p
            pos += len(toks)
        per_agent.append(rows)

    n = len(agents)
    n_dedup = len(ids)
    m = [len(r) for r in per_agent]
    maxlb = max(m) if m else 0
    block_table = np.full((n, maxlb), -1, np.int32)
    delta_table = np.full((n, maxlb), -1, np.int32)
    ntok = np.zeros((n, maxlb), np.int32)
    dst_pos0 = np.zeros((n, maxlb), np.int32)
    shift = np.zeros((n, maxlb), np.int32)
    for j, rows in enumerate(per_agent):
        for b, (p, nt, d0, _, _) in enumerate(rows):
            block_table[j, b] = p
            ntok[j, b] = nt
            dst_pos0[j, b] = d0
            shift[j, b] = d0 - src_pos0[p]

    # deltas: validate, then number them after the dedup ids in (j, b) order
    next_id = n_dedup
    for j, ag in enumerate(agents):
        db = [int(x) for x in ag.delta_blocks]
        for i, b in enumerate(db):
            if b < 0 or b >= m[j] or (i and db[i - 1] >= b):
                raise OracleError(EINVAL, "delta index out of range or unsorted")
            _, _, _, kind, tier = per_agent[j][b]
            if kind != SEGMENT or tier == PRIVATE:
                raise OracleError(EINVAL, "delta on a block that is not a shared segment block")
        for b in db:
            master = int(block_table[j, b])
            delta_table[j, b] = next_id
            src_pos0.append(src_pos0[master])
            phys_ntok.append(int(ntok[j, b]))
            phys_agent.append(j)
            phys_block.append(b)
            next_id += 1

    n_phys = next_id
    refcount = np.zeros(n_phys, np.int32)
    for j in range(n):
        for b in range(m[j]):
            e = delta_table[j, b] if delta_table[j, b] >= 0 else block_table[j, b]
            refcount[e] += 1

    return dict(
        n_agents=n, max_blocks=maxlb, n_dedup=n_dedup, n_delta=n_phys - n_dedup, n_phys=n_phys,
        n_blocks=np.array(m, np.int32), block_table=block_table, delta_table=delta_table,
        ntok=ntok, dst_pos0=dst_pos0, shift=shift,
        src_pos0=np.array(src_pos0, np.int32), refcount=refcount,
        phys_ntok=np.array(phys_ntok, np.int32), phys_agent=np.array(phys_agent, np.int32),
        phys_block=np.array(phys_block, np.int32),
    )


def unique_kv_bytes(tables: dict, n_kv_heads: int, head_dim: int, kv_dtype: int, n_layers: int = 1) -> int:
    """Bytes of the physical pool that hold valid tokens: per valid token and kv
    head, K and V each take head_dim bf16 values, or head_dim/2 code bytes plus one
    (fp16 scale, fp16 zero) pair per 64 elements for Q4."""
    tok = int(tables["phys_ntok"].astype(np.int64).sum())
    if kv_dtype == 0:
        per = 2 * head_dim * 2
    else:
        per = 2 * (head_dim // 2 + (head_dim // 64) * 4)
    return tok * n_kv_heads * per * n_layers
