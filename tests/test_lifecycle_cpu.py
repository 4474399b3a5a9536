"""Block lifecycle (append with copy-on-write, destroy, lose, audit, reclaim) on
the CPU.  First the oracle replay is pinned by closed forms, invariants and
brute force; then the library's host calls are compared with it bit for bit
over seeded random operation sequences, including pool-full and error cases."""
import ctypes as C

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import dedup
from oracle import lifecycle as olc
from shared_paged_kv_amd import _lib as K
from tests.test_tables_cpu import check_plan_coverage
from workload import spec

SNAP_KEYS = ["n_blocks", "block_table", "delta_table", "ntok", "dst_pos0", "shift", "src_pos0", "refcount",
             "phys_ntok"]


def _agents_shared_tail(n_agents, n_tok, tier=spec.GROUP):
    toks = (np.arange(n_tok, dtype=np.int32) * 7919 + 11) % (1 << 29) + 1
    return [spec.Agent([spec.Span(tier, 0, spec.PREFIX, toks.copy())]) for _ in range(n_agents)]


# ---------------------------------------------------------------------------
# oracle pins


def test_oracle_shared_partial_block_closed_form():
    """k agents share a partial last block: one append each makes k - 1 copies
    (the last writer is then the only holder and writes in place); the copies
    take the next ids in call order; later appends copy nothing until the
    blocks fill, then each agent gets one new block of its own."""
    k, B = 5, 16
    agents = _agents_shared_tail(k, 40)          # blocks of 16, 16, 8 tokens, shared by all
    t = dedup.build_tables(B, agents)
    assert t["n_phys"] == 3 and list(t["refcount"]) == [k, k, k]
    r = olc.PoolReplay(t, B, capacity=64)
    copies, writes = r.append(list(range(k)))
    assert copies == [(2, 3 + i) for i in range(k - 1)]
    assert writes == [(3 + i, 8, i, 0) for i in range(k - 1)] + [(2, 8, k - 1, 0)]
    assert r.refcount[2] == 1 and all(r.refcount[3 + i] == 1 for i in range(k - 1))
    for step in range(7):                        # slots 9..15: in place everywhere
        copies, writes = r.append(list(range(k)))
        assert copies == [] and [w[1] for w in writes] == [9 + step] * k
    copies, writes = r.append(list(range(k)))    # every last block is full now
    new = [w[0] for w in writes]
    assert copies == [] and new == list(range(3 + k - 1, 3 + 2 * k - 1))
    tb = r.tables()
    assert all(int(tb["dst_pos0"][j, 3]) == 48 and int(tb["ntok"][j, 3]) == 1 for j in range(k))
    assert sum(tb["refcount"]) == sum(int(x) for x in tb["n_blocks"])


def test_oracle_private_tail_never_copies():
    """Agents whose last block is private (count 1) write in place; new blocks
    only when a block fills; ids in call order."""
    wl = spec.make("tiny")
    t = dedup.build_tables(wl.shape.block_tokens, wl.agents)
    r = olc.PoolReplay(t, wl.shape.block_tokens, capacity=t["n_phys"] + 64)
    n = wl.n_agents
    total_new = 0
    for _ in range(40):
        copies, writes = r.append(list(range(n)))
        assert copies == []
        total_new += sum(1 for w in writes if w[1] == 0)
    assert r.high == t["n_phys"] + total_new
    tb = r.tables()
    for j in range(n):
        assert int(tb["ntok"][j, : tb["n_blocks"][j]].sum()) == wl.context_len(j) + 40


def _check_invariants(r):
    tb = r.tables()
    rc = r.recount()
    live_refs = sum(len(rows) for j, rows in enumerate(r.entries) if r.alive[j] == "live")
    assert sum(rc) == live_refs
    for p in range(r.high):
        if r.used[p]:
            assert r.phys_ntok[p] >= 1
        else:
            assert r.refcount[p] == 0
    # every live entry's block holds exactly the entry's tokens
    for j, rows in enumerate(r.entries):
        for e in rows:
            assert r.used[r._eff(e)] and r.phys_ntok[r._eff(e)] == e[3]
    return tb


def test_oracle_random_ops_invariants_and_token_counts():
    wl = spec.make("tiny_seg")
    B = wl.shape.block_tokens
    t = dedup.build_tables(B, wl.agents)
    r = olc.PoolReplay(t, B, capacity=t["n_phys"] + 200)
    g = np.random.default_rng(3)
    length = [wl.context_len(j) for j in range(wl.n_agents)]
    for _ in range(60):
        live = [j for j in range(wl.n_agents) if r.alive[j] == "live"]
        if not live:
            break
        if g.random() < 0.92:
            sel = list(g.choice(live, size=int(g.integers(1, 2 * len(live) + 1))))
            r.append(sel)
            for j in sel:
                length[j] += 1
        else:
            r.destroy(int(g.choice(live)))
        assert r.audit()["n_mismatched"] == 0
        tb = _check_invariants(r)
        for j in range(wl.n_agents):
            if r.alive[j] == "live":
                assert int(tb["ntok"][j, : tb["n_blocks"][j]].sum()) == length[j]


def test_oracle_destroy_all_frees_every_block():
    wl = spec.make("small_round")
    B = wl.shape.block_tokens
    t = dedup.build_tables(B, wl.agents)
    r = olc.PoolReplay(t, B, capacity=t["n_phys"] + 64)
    r.append(list(range(wl.n_agents)))
    for j in range(wl.n_agents):
        r.destroy(j)
    a = r.audit()
    assert a["n_allocated"] == 0 and a["n_live_agents"] == 0 and a["n_mismatched"] == 0


def test_oracle_lost_agent_leaks_exactly_its_sole_blocks():
    """Brute force: the leaked blocks of a lost agent are the blocks no other
    live agent references; reclaim frees exactly them."""
    wl = spec.make("small_round")
    B = wl.shape.block_tokens
    t = dedup.build_tables(B, wl.agents)
    r = olc.PoolReplay(t, B, capacity=t["n_phys"] + 64)
    r.append([0, 1, 2, 3, 1])
    j = 1
    mine = {r._eff(e) for e in r.entries[j]}
    others = {r._eff(e) for i, rows in enumerate(r.entries) if i != j for e in rows}
    sole = sorted(mine - others)
    toks = sum(r.phys_ntok[p] for p in sole)
    r.lose(j)
    a = r.audit()
    assert a["leaked_ids"] == sole and a["n_leaked"] == len(sole) and a["leaked_tokens"] == toks
    assert a["n_mismatched"] == len(mine)
    assert r.reclaim() == len(sole)
    a = r.audit()
    assert a["n_leaked"] == 0 and a["n_mismatched"] == 0


def test_oracle_full_pool_changes_nothing():
    k, B = 4, 16
    t = dedup.build_tables(B, _agents_shared_tail(k, 40))
    r = olc.PoolReplay(t, B, capacity=t["n_phys"] + 2)
    before = r.tables()
    with pytest.raises(olc.PoolFull):
        r.append(list(range(k)))                 # needs k - 1 = 3 copies
    after = r.tables()
    for key in SNAP_KEYS:
        assert np.array_equal(before[key], after[key]), key
    copies, _ = r.append([0, 1])                 # 2 copies fit
    assert len(copies) == 2


def test_oracle_content_model_brute_force():
    """After appends, each agent's dense context from the content model is its
    original dense context (oracle.attention) followed by the appended rows:
    K within two bf16 rounding steps of the given rows (exact where unshifted),
    V exact."""
    wl = spec.make("tiny_seg")
    sh = wl.shape
    B = sh.block_tokens
    t = dedup.build_tables(B, wl.agents)
    store = oatt._Store(wl, 0)
    kvh = list(range(sh.n_kv_heads))
    orig = [oatt.dense_from_tables(wl, t, j, store, kvh) for j in range(wl.n_agents)]
    r = olc.PoolReplay(t, B, capacity=t["n_phys"] + 64)

    def stored(p):
        j, b = int(t["phys_agent"][p]), int(t["phys_block"][p])
        seed = wl.blk_delta_seed[j][b] if p >= t["n_dedup"] else wl.blk_seed[j][b]
        nt = int(t["phys_ntok"][p])
        K = np.stack([store.get(seed, nt, g)[0] for g in kvh], 1)
        V = np.stack([store.get(seed, nt, g)[1] for g in kvh], 1)
        return K, V

    r.model_contents(stored)
    g = np.random.default_rng(5)
    added = {j: ([], []) for j in range(wl.n_agents)}
    for _ in range(20):
        sel = [int(x) for x in g.integers(0, wl.n_agents, size=3)]
        kr = olc.bf16_round(g.standard_normal((3, sh.n_kv_heads, sh.head_dim)))
        vr = olc.bf16_round(g.standard_normal((3, sh.n_kv_heads, sh.head_dim)))
        r.append(sel, kr, vr, sh.rope_theta)
        for i, j in enumerate(sel):
            added[j][0].append(kr[i])
            added[j][1].append(vr[i])
    for j in range(wl.n_agents):
        Kd, Vd = r.dense(j, sh.rope_theta)
        K0, V0 = orig[j]
        n0 = K0.shape[0]
        assert np.array_equal(Kd[:n0], K0) and np.array_equal(Vd[:n0], V0)
        if added[j][0]:
            ka, va = np.array(added[j][0], np.float64), np.array(added[j][1], np.float64)
            assert np.array_equal(Vd[n0:], va)
            # one bf16 rounding of the stored rotated pair (half an ulp of each
            # element, bounded by 2^-8 of the pair's norm), rotated back exactly
            h = sh.head_dim // 2
            pair = np.sqrt(ka[..., :h] ** 2 + ka[..., h:] ** 2)
            bound = np.concatenate([pair, pair], -1) * 2.0 ** -8 * 1.0001
            assert np.all(np.abs(Kd[n0:] - ka) <= bound)


# ---------------------------------------------------------------------------
# library against the oracle


def _snap_same(pool, r):
    S = pool.tables().arrays
    O = r.tables()
    for k in SNAP_KEYS:
        assert np.array_equal(S[k], O[k]), k
    assert S["n_phys"] == O["n_phys"]
    return S


def _audit_same(pool, r):
    a, o = pool.audit(max_ids=4096), r.audit()
    for k in ("n_allocated", "n_leaked", "n_mismatched", "n_live_agents", "leaked_tokens"):
        assert a[k] == o[k], k
    assert list(a["leaked_ids"]) == o["leaked_ids"]


@pytest.mark.parametrize("name,extra", [("tiny_seg", 40), ("small_round", 12), ("tiny", 300), ("tiny_q4", 60),
                                        ("round_b256", 20)])
def test_lifecycle_bit_exact_random_ops(name, extra):
    wl = spec.small_round(block_tokens=256) if name == "round_b256" else spec.make(name)
    B = wl.shape.block_tokens
    T = K.build_tables(wl.shape, wl.agents)
    t = dedup.build_tables(B, wl.agents)
    cap = T.n_phys + extra
    pool = K.BlockPool(T, wl.shape, cap)
    r = olc.PoolReplay(t, B, cap)
    grp = wl.shape.n_q_heads // wl.shape.n_kv_heads
    g = np.random.default_rng(11)
    n_full = 0
    for step in range(80):
        live = [j for j in range(wl.n_agents) if r.alive[j] == "live"]
        u = g.random()
        if not live:
            break
        if u < 0.75:
            sel = [int(x) for x in g.choice(live, size=int(g.integers(1, 3 * len(live) + 1)))]
            try:
                oc, ow = r.append(sel)
            except olc.PoolFull:
                with pytest.raises(K.KvpError) as ei:
                    pool.append(sel)
                assert ei.value.code == K.KVP_EFULL
                n_full += 1
            else:
                lc, lw = pool.append(sel)
                assert [tuple(x) for x in lc.tolist()] == oc
                assert [tuple(x) for x in lw.tolist()] == ow
        elif u < 0.85:
            j = int(g.choice(live))
            r.destroy(j)
            pool.destroy(j)
        elif u < 0.92:
            j = int(g.choice(live))
            r.lose(j)
            pool.lose(j)
        else:
            assert pool.reclaim() == r.reclaim()
        S = _snap_same(pool, r)
        _audit_same(pool, r)
        if step % 8 == 0:
            check_plan_coverage(S, grp)
    assert n_full >= 0


def test_full_pool_library_matches_oracle():
    """The append that needs more blocks than the pool has left fails with
    KVP_EFULL and changes nothing; a smaller one then succeeds identically."""
    k, B = 4, 16
    agents = _agents_shared_tail(k, 40)
    shape = spec.Shape(1, 2, 1, 64, B, spec.BF16, 1e4)
    T = K.build_tables(shape, agents)
    t = dedup.build_tables(B, agents)
    pool = K.BlockPool(T, shape, T.n_phys + 2)
    r = olc.PoolReplay(t, B, T.n_phys + 2)
    with pytest.raises(K.KvpError) as ei:
        pool.append(list(range(k)))
    assert ei.value.code == K.KVP_EFULL
    with pytest.raises(olc.PoolFull):
        r.append(list(range(k)))
    _snap_same(pool, r)
    lc, lw = pool.append([0, 1])
    oc, ow = r.append([0, 1])
    assert [tuple(x) for x in lc.tolist()] == oc and [tuple(x) for x in lw.tolist()] == ow
    _snap_same(pool, r)


def test_lifecycle_errors():
    wl = spec.make("tiny_seg")
    T = K.build_tables(wl.shape, wl.agents)
    with pytest.raises(K.KvpError) as ei:
        K.BlockPool(T, wl.shape, T.n_phys - 1)
    assert ei.value.code == K.KVP_EINVAL
    pool = K.BlockPool(T, wl.shape, T.n_phys + 8)
    for bad in ([wl.n_agents], [-1], [0, 99]):
        with pytest.raises(K.KvpError) as ei:
            pool.append(bad)
        assert ei.value.code == K.KVP_EINVAL
    pool.destroy(1)
    for call in (lambda: pool.append([1]), lambda: pool.destroy(1), lambda: pool.lose(1)):
        with pytest.raises(K.KvpError) as ei:
            call()
        assert ei.value.code == K.KVP_EINVAL
    # nothing changed by the failed calls
    r = olc.PoolReplay(dedup.build_tables(wl.shape.block_tokens, wl.agents), wl.shape.block_tokens, T.n_phys + 8)
    r.destroy(1)
    _snap_same(pool, r)
    L = K.lib()
    au = K.kvp_audit()
    assert L.kvpool_audit(None, C.byref(au), None, 0) == K.KVP_EINVAL
    assert L.kvpool_audit(pool._h, C.byref(au), None, -1) == K.KVP_EINVAL
    assert L.kvpool_reclaim(None) == K.KVP_EINVAL
    assert L.kvpool_pool_tables(None, None) == K.KVP_EINVAL
    ops = K.kvp_append_ops()
    assert L.kvpool_append(pool._h, 2, None, C.byref(ops)) == K.KVP_EINVAL


def test_kv_append_argument_errors_without_launch():
    wl = spec.make("tiny_seg")
    sh = K.make_shape(wl.shape)
    L = K.lib()
    one = C.c_void_p(1)
    assert L.kv_append(None, one, one, 8, None, 0, None, 0, None, None, 0, None) == K.KVP_EINVAL
    assert L.kv_append(C.byref(sh), one, one, 0, None, 0, None, 0, None, None, 0, None) == K.KVP_EINVAL
    assert L.kv_append(C.byref(sh), one, one, 8, None, 1, None, 0, None, None, 0, None) == K.KVP_EINVAL
    assert L.kv_append(C.byref(sh), one, one, 8, None, 0, one, 1, None, None, 1, None) == K.KVP_EINVAL
    assert L.kv_append(C.byref(sh), None, one, 8, one, 1, None, 0, None, None, 0, None) == K.KVP_EINVAL
    q4 = K.make_shape(spec.make("tiny_q4").shape)
    assert L.kv_append(C.byref(q4), one, one, 8, None, 0, None, 0, None, None, 0, None) == K.KVP_EINVAL
