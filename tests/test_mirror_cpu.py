"""Master/mirror diff construction and restore on the CPU: the oracle
(oracle/mirror.py) pinned by closed forms, brute force and the sharing
invariance, and the library's restore list bit-exact with the oracle tables."""
import numpy as np
import pytest

from oracle import attention as oatt
from oracle import dedup
from oracle import mirror as omir
from shared_paged_kv_amd import _lib as K
from workload import rng, spec


def _rand_bits(g, shape):
    return rng.f32_to_bf16_bits(g.standard_normal(shape).astype(np.float32))


def test_diff_flags_closed_forms():
    g = np.random.default_rng(1)
    n, L, H, B, d = 6, 2, 2, 16, 8
    mk, mv = _rand_bits(g, (n, L, H, B, d)), _rand_bits(g, (n, L, H, B, d))
    ck, cv = mk.copy(), mv.copy()
    ntok = np.array([16, 16, 9, 9, 16, 5])
    ck[1, 1, 0, 3, 2] ^= 1                      # one bit of one valid K value
    cv[2, 0, 1, 12, 0] ^= 0x40                  # a padding slot of a 9-token block: ignored
    mv[3, 0, 1, 8, 7], cv[3, 0, 1, 8, 7] = 0x3F00, 0x4000   # last valid slot of a 9-token block: 0.5 -> 2
    mk[4, 0, 0, 0, 0], ck[4, 0, 0, 0, 0] = 0x3F00, 0x3F40   # 0.5 -> 0.75: a change of exactly 0.25
    cv[5, 0, 0, 4, 0] = 0x7FC0                  # NaN in a valid slot
    assert list(omir.diff_flags(mk, mv, ck, cv, ntok, 0.0)) == [0, 1, 0, 1, 1, 1]
    # threshold: the 0.25 change differs for tau < 0.25 only; a NaN always differs
    f = omir.diff_flags(mk, mv, ck, cv, ntok, 0.25)
    assert list(f) == [0, 0, 0, 1, 0, 1]
    assert omir.diff_flags(mk, mv, ck, cv, ntok, 0.2)[4] == 1


def test_diff_flags_brute_force():
    g = np.random.default_rng(2)
    n, L, H, B, d = 20, 2, 2, 4, 4
    mk, mv = _rand_bits(g, (n, L, H, B, d)), _rand_bits(g, (n, L, H, B, d))
    ck, cv = mk.copy(), mv.copy()
    ntok = g.integers(1, B + 1, n)
    for i in range(n):
        if g.random() < 0.5:
            idx = tuple(int(g.integers(0, s)) for s in (L, H, B, d))
            (ck if g.random() < 0.5 else cv)[(i,) + idx] ^= np.uint16(1 << int(g.integers(0, 15)))
    for tau in (0.0, 1e-3, 0.5):
        want = []
        for i in range(n):
            w = 0
            for a, b in ((mk[i], ck[i]), (mv[i], cv[i])):
                for l in range(L):
                    for h in range(H):
                        for t in range(int(ntok[i])):
                            for e in range(d):
                                if tau == 0:
                                    w |= int(a[l, h, t, e] != b[l, h, t, e])
                                else:
                                    fa = np.float32(omir.bf16_bits_to_f64(a[l, h, t, e]))
                                    fb = np.float32(omir.bf16_bits_to_f64(b[l, h, t, e]))
                                    w |= int(not abs(fa - fb) <= np.float32(tau))
            want.append(w)
        assert list(omir.diff_flags(mk, mv, ck, cv, ntok, tau)) == want


@pytest.mark.parametrize("name", ["tiny_seg", "small_round"])
def test_restore_matches_logical_context(name):
    """The restored valid tokens of every agent are its logical context (dense
    from the workload's own description, keys rounded to bf16 where moved): the
    gather through the tables loses nothing; padding slots are zero."""
    wl = spec.make(name)
    sh = wl.shape
    t = dedup.build_tables(sh.block_tokens, wl.agents)
    store = oatt._Store(wl, 0)
    kvh = list(range(sh.n_kv_heads))

    def stored(p):
        j, b = int(t["phys_agent"][p]), int(t["phys_block"][p])
        seed = wl.blk_delta_seed[j][b] if p >= t["n_dedup"] else wl.blk_seed[j][b]
        nt = int(t["phys_ntok"][p])
        return (np.stack([store.get(seed, nt, g)[0] for g in kvh], 1),
                np.stack([store.get(seed, nt, g)[1] for g in kvh], 1))

    for j in range(wl.n_agents):
        Kr, Vr = omir.restore_blocks(t, j, stored, sh.block_tokens, sh.rope_theta)
        Kp, Vp = oatt.dense_plain(wl, j, store, kvh)
        nt = [int(x) for x in t["ntok"][j, : t["n_blocks"][j]]]
        Kv = np.concatenate([Kr[b, :n] for b, n in enumerate(nt)])
        Vv = np.concatenate([Vr[b, :n] for b, n in enumerate(nt)])
        assert np.array_equal(Vv, Vp)
        shifted = np.concatenate([np.full(n, t["shift"][j, b] != 0) for b, n in enumerate(nt)])
        assert np.array_equal(Kv[~shifted], Kp[~shifted])
        h = sh.head_dim // 2
        pair = np.sqrt(Kp[shifted][..., :h] ** 2 + Kp[shifted][..., h:] ** 2)
        assert np.all(np.abs(Kv[shifted] - Kp[shifted]) <= np.concatenate([pair, pair], -1) * 2.0 ** -8 * 1.0001)
        for b, n in enumerate(nt):
            assert not Kr[b, n:].any() and not Vr[b, n:].any()


@pytest.mark.parametrize("name", ["tiny_seg", "small_round", "tokendance"])
def test_restore_list_matches_oracle_tables(name):
    """Per agent and for a list of agents (with a repeat): the entries, put in
    destination order, are each logical block's (delta else master, shift,
    valid tokens); the list is ordered by (source, valid tokens, shift, dest)."""
    wl = spec.make(name)
    T = K.build_tables(wl.shape, wl.agents)
    t = dedup.build_tables(wl.shape.block_tokens, wl.agents)

    def want_of(j):
        m = int(t["n_blocks"][j])
        eff = np.where(t["delta_table"][j, :m] >= 0, t["delta_table"][j, :m], t["block_table"][j, :m])
        return np.stack([eff, t["shift"][j, :m], t["ntok"][j, :m]], 1)

    lists = [[j] for j in range(wl.n_agents)] + [[wl.n_agents - 1, 0, wl.n_agents - 1]]
    for agents in lists:
        got = K.restore_list(T, agents)
        want = np.concatenate([want_of(j) for j in agents])
        assert len(got) == len(want)
        assert sorted(got[:, 3].tolist()) == list(range(len(want)))
        by_dst = got[np.argsort(got[:, 3])]
        assert np.array_equal(by_dst[:, :3], want)
        keys = [tuple(r) for r in got[:, [0, 2, 1, 3]].tolist()]
        assert keys == sorted(keys)
    assert len(K.restore_list(T, [])) == 0


def test_mirror_argument_errors_without_launch():
    import ctypes as C
    wl = spec.make("tiny_seg")
    sh = K.make_shape(wl.shape)
    L = K.lib()
    one = C.c_void_p(1)
    assert L.kv_restore(None, one, one, 8, one, 1, one, one, 8, None) == K.KVP_EINVAL
    assert L.kv_restore(C.byref(sh), one, one, 0, one, 1, one, one, 8, None) == K.KVP_EINVAL
    assert L.kv_restore(C.byref(sh), one, one, 8, one, 1, one, one, 0, None) == K.KVP_EINVAL
    assert L.kv_restore(C.byref(sh), one, one, 8, None, 1, one, one, 8, None) == K.KVP_EINVAL
    assert L.kv_restore(C.byref(sh), one, one, 8, one, -1, one, one, 8, None) == K.KVP_EINVAL
    assert L.kv_diff_blocks(C.byref(sh), one, one, 8, one, one, 8, one, 1, -1.0, one, None) == K.KVP_EINVAL
    assert L.kv_diff_blocks(C.byref(sh), one, one, 8, one, one, 8, one, 1, float("nan"), one, None) == K.KVP_EINVAL
    assert L.kv_diff_blocks(C.byref(sh), one, one, 8, one, one, 0, one, 1, 0.0, one, None) == K.KVP_EINVAL
    assert L.kv_diff_blocks(C.byref(sh), one, one, 8, one, one, 8, None, 1, 0.0, one, None) == K.KVP_EINVAL
    q4 = K.make_shape(spec.make("tiny_q4").shape)
    assert L.kv_restore(C.byref(q4), one, one, 8, one, 1, one, one, 8, None) == K.KVP_EINVAL
    T = K.build_tables(wl.shape, wl.agents)
    P32 = C.POINTER(C.c_int32)
    bad = (C.c_int32 * 1)(wl.n_agents)
    good = (C.c_int32 * 1)(0)
    assert L.kvpool_restore_list(T._h, C.cast(bad, P32), 1, None, 0) == K.KVP_EINVAL
    assert L.kvpool_restore_list(T._h, C.cast(good, P32), 1, None, 4) == K.KVP_EINVAL
    assert L.kvpool_restore_list(T._h, None, 1, None, 0) == K.KVP_EINVAL
    assert L.kvpool_restore_list(T._h, C.cast(good, P32), -1, None, 0) == K.KVP_EINVAL
    assert L.kvpool_restore_list(None, C.cast(good, P32), 1, None, 0) == K.KVP_EINVAL
    # too small a buffer: the size comes back, nothing is written
    n = L.kvpool_restore_list(T._h, C.cast(good, P32), 1, None, 0)
    buf = (C.c_int32 * (4 * n))(*([-7] * (4 * n)))
    assert L.kvpool_restore_list(T._h, C.cast(good, P32), 1, C.cast(buf, P32), n - 1) == n
    assert list(buf) == [-7] * (4 * n)
