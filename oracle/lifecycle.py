"""Block lifecycle replay: append with copy-on-write, destroy, leak audit (oracle).

INMS walkthrough, sec. 2.2: shared blocks are read-only; a sequence about to
write into a block whose reference count is above one is given its own copy of
that block first (the old block's count drops by one), otherwise it writes in
place.  Sec. 3.3: destroying a sequence decrements the counts of its blocks and
returns the blocks that reach zero.  Sec. 5.3: an agent that exits without its
destroy call leaves its counts behind (a leak); a periodic scan finds the blocks
nobody references and a forced reclamation returns them.

This is a plain Python replay of those rules over the tables of
``oracle.dedup.build_tables``, plus a content model (per physical block, the
stored K and V of every slot, float64) so that decode attention after appends
can be recomputed densely.

Readings taken where the pages are silent (the same list is in the design notes):
* one appended token goes to the agent's last logical block while it holds
  fewer than B tokens, else to a new logical block placed right after it;
* a copy keeps the source's stored frame (src_pos0) and contents; a new block's
  frame is the logical position of its first token;
* the token's K is given post-RoPE at its logical position; it is stored in the
  block's frame, R(-shift) k rounded to bf16 (nearest even); V as given;
* a freed id is reused smallest first, otherwise the smallest id never used;
  ids stay below the pool's capacity ("full" otherwise; the call then changes
  nothing);
* an entry overlaid by a delta writes into the delta block (count 1);
* an overlaid entry keeps naming its master only while that very allocation is
  alive; afterwards the entry is the delta block alone.
"""
from __future__ import annotations

import copy

import numpy as np

from . import rope as _rope


class PoolFull(RuntimeError):
    pass


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even), returned as float64."""
    f = np.asarray(x, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


class PoolReplay:
    """tables: dict from oracle.dedup.build_tables; B: block tokens."""

    def __init__(self, tables: dict, B: int, capacity: int):
        n_phys = int(tables["n_phys"])
        if capacity < n_phys:
            raise ValueError("capacity below the tables' physical blocks")
        self.B, self.capacity = int(B), int(capacity)
        self.refcount = [0] * capacity
        self.src_pos0 = [0] * capacity
        self.phys_ntok = [0] * capacity
        self.serial = [0] * capacity      # which allocation an id currently holds
        self.used = [False] * capacity
        self.next_serial = 1
        for p in range(n_phys):
            self.refcount[p] = int(tables["refcount"][p])
            self.src_pos0[p] = int(tables["src_pos0"][p])
            self.phys_ntok[p] = int(tables["phys_ntok"][p])
            self.serial[p] = self.next_serial
            self.next_serial += 1
            self.used[p] = self.refcount[p] > 0
            if not self.used[p]:
                self.phys_ntok[p] = 0
        self.high = n_phys                 # ids >= high were never handed out
        self.alive = []                    # "live" | "destroyed" | "lost"
        self.entries = []                  # per agent: list of [table, serial, delta, ntok, dst_pos0]
        for j in range(int(tables["n_agents"])):
            rows = []
            for b in range(int(tables["n_blocks"][j])):
                p = int(tables["block_table"][j, b])
                rows.append([p, self.serial[p], int(tables["delta_table"][j, b]),
                             int(tables["ntok"][j, b]), int(tables["dst_pos0"][j, b])])
            self.entries.append(rows)
            self.alive.append("live")
        self.content = {}   # physical id -> (K [ntok, Hkv, d], V) float64, when modelled

    # -- helpers --------------------------------------------------------------
    @staticmethod
    def _eff(e):
        return e[2] if e[2] >= 0 else e[0]

    def _take_id(self):
        free = [p for p in range(self.high) if not self.used[p]]
        if free:
            p = free[0]
        elif self.high < self.capacity:
            p = self.high
            self.high += 1
        else:
            raise PoolFull("no free physical block")
        self.used[p] = True
        self.serial[p] = self.next_serial
        self.next_serial += 1
        self.refcount[p] = 0
        self.phys_ntok[p] = 0
        return p

    def _release(self, p):
        self.used[p] = False
        self.refcount[p] = 0
        self.phys_ntok[p] = 0

    # -- lifecycle ------------------------------------------------------------
    def append(self, agents, k_rows=None, v_rows=None, base=None):
        """One token per listed agent, in order.  With k_rows / v_rows (float64
        [n, Hkv, d] per listed agent, bf16 values) and the RoPE base, the content
        model is updated too (blocks whose contents are not modelled are only
        bookkept).  Returns (copies [(src, dst)], writes [(id, slot,
        row, shift)])."""
        saved = copy.deepcopy((self.refcount, self.src_pos0, self.phys_ntok, self.serial, self.used,
                               self.next_serial, self.high, self.entries, self.content))
        copies, writes = [], []
        try:
            for row, j in enumerate(agents):
                if not (0 <= j < len(self.entries)) or self.alive[j] != "live":
                    raise ValueError("agent out of range or not live")
                rows = self.entries[j]
                if not rows or rows[-1][3] >= self.B:
                    pos = rows[-1][4] + rows[-1][3] if rows else 0
                    q = self._take_id()
                    self.refcount[q] = 1
                    self.src_pos0[q] = pos
                    rows.append([q, self.serial[q], -1, 0, pos])
                    if k_rows is not None:
                        empty = np.zeros((0,) + np.shape(k_rows[row]), np.float64)
                        self.content[q] = (empty, empty.copy())
                    target = q
                else:
                    e = rows[-1]
                    target = self._eff(e)
                    if self.refcount[target] > 1:
                        q = self._take_id()
                        self.refcount[target] -= 1
                        self.refcount[q] = 1
                        self.src_pos0[q] = self.src_pos0[target]
                        self.phys_ntok[q] = self.phys_ntok[target]
                        if target in self.content:
                            K, V = self.content[target]
                            self.content[q] = (K.copy(), V.copy())
                        copies.append((target, q))
                        e[0], e[1], e[2] = q, self.serial[q], -1
                        target = q
                e = rows[-1]
                slot = e[3]
                shift = e[4] - self.src_pos0[target]
                writes.append((target, slot, row, shift))
                e[3] += 1
                self.phys_ntok[target] = e[3]
                if k_rows is not None and target in self.content:
                    K, V = self.content[target]
                    k = bf16_round(_rope.rotate(k_rows[row], -shift, base)) if shift else np.asarray(k_rows[row], np.float64)
                    K = np.concatenate([K[:slot], k[None]], 0)
                    V = np.concatenate([V[:slot], np.asarray(v_rows[row], np.float64)[None]], 0)
                    self.content[target] = (K, V)
        except Exception:
            (self.refcount, self.src_pos0, self.phys_ntok, self.serial, self.used,
             self.next_serial, self.high, self.entries, self.content) = saved
            raise
        return copies, writes

    def destroy(self, j):
        if not (0 <= j < len(self.entries)) or self.alive[j] != "live":
            raise ValueError("agent out of range or not live")
        for e in self.entries[j]:
            p = self._eff(e)
            self.refcount[p] -= 1
            if self.refcount[p] == 0:
                self._release(p)
        self.entries[j] = []
        self.alive[j] = "destroyed"

    def lose(self, j):
        if not (0 <= j < len(self.entries)) or self.alive[j] != "live":
            raise ValueError("agent out of range or not live")
        self.entries[j] = []
        self.alive[j] = "lost"

    def recount(self):
        rc = [0] * self.capacity
        for j, rows in enumerate(self.entries):
            if self.alive[j] == "live":
                for e in rows:
                    rc[self._eff(e)] += 1
        return rc

    def audit(self):
        rc = self.recount()
        held = [p for p in range(self.high) if self.used[p]]
        leaked = [p for p in held if self.refcount[p] > 0 and rc[p] == 0]
        return dict(n_allocated=len(held), n_leaked=len(leaked),
                    n_mismatched=sum(1 for p in held if self.refcount[p] != rc[p]),
                    n_live_agents=sum(1 for s in self.alive if s == "live"),
                    leaked_tokens=sum(self.phys_ntok[p] for p in leaked), leaked_ids=leaked)

    def reclaim(self):
        rc = self.recount()
        freed = 0
        for p in range(self.high):
            if self.used[p]:
                self.refcount[p] = rc[p]
                if rc[p] == 0:
                    self._release(p)
                    freed += 1
        return freed

    # -- views ----------------------------------------------------------------
    def tables(self) -> dict:
        n = len(self.entries)
        m = [len(r) for r in self.entries]
        M = max(m) if m else 0
        bt = np.full((n, M), -1, np.int32)
        dt = np.full((n, M), -1, np.int32)
        nt = np.zeros((n, M), np.int32)
        d0 = np.zeros((n, M), np.int32)
        sh = np.zeros((n, M), np.int32)
        for j, rows in enumerate(self.entries):
            for b, (t, ser, d, ntok, pos) in enumerate(rows):
                master_alive = d >= 0 and self.used[t] and self.serial[t] == ser
                bt[j, b] = d if (d >= 0 and not master_alive) else t
                dt[j, b] = d if master_alive else -1
                nt[j, b] = ntok
                d0[j, b] = pos
                sh[j, b] = pos - self.src_pos0[self._eff([t, ser, d])]
        # the whole pool, capacity ids (never-used and freed ids: no tokens, count 0)
        C_ = self.capacity
        return dict(n_agents=n, max_blocks=M, n_phys=C_, n_blocks=np.array(m, np.int32), block_table=bt,
                    delta_table=dt, ntok=nt, dst_pos0=d0, shift=sh,
                    src_pos0=np.array(self.src_pos0, np.int32),
                    refcount=np.array([self.refcount[p] if self.used[p] else 0 for p in range(C_)], np.int32),
                    phys_ntok=np.array([self.phys_ntok[p] if self.used[p] else 0 for p in range(C_)], np.int32))

    # -- content model ----------------------------------------------------------
    def model_contents(self, stored):
        """stored(p) -> (K [ntok, Hkv, d], V) float64 stored-frame contents of
        original block p; called for every block an agent reads now."""
        for rows in self.entries:
            for e in rows:
                p = self._eff(e)
                if p not in self.content:
                    K, V = stored(p)
                    self.content[p] = (np.asarray(K, np.float64), np.asarray(V, np.float64))

    def dense(self, j, base):
        """Agent j's dense context (K moved to its logical positions, V) from the
        content model: K, V [L, Hkv, d] float64."""
        Ks, Vs = [], []
        for e in self.entries[j]:
            p = self._eff(e)
            K, V = self.content[p]
            K, V = K[:e[3]], V[:e[3]]
            shift = e[4] - self.src_pos0[p]
            Ks.append(_rope.rotate(K, shift, base) if shift else K)
            Vs.append(V)
        if not Ks:
            return None, None
        return np.concatenate(Ks, 0), np.concatenate(Vs, 0)
