"""Master/mirror steps on the GPU through the C ABI: kv_restore against the
oracle's restore (V and unrotated K bit-exact, rotated K within one bf16 ulp,
padding zero), the fused restore bit-identical to the three-pass one it
replaces (copy the masters, overwrite the deltas, re-rotate), and
kv_diff_blocks against the oracle's flags -- planted differences, the threshold,
padding, bad entries, and the delta lists of a built round recovered from the
agents' blocks."""
import numpy as np
import pytest

from oracle import dedup
from oracle import mirror as omir
from shared_paged_kv_amd import _lib as K
from workload import device as wdev
from workload import spec

from .gpu_util import log

pytestmark = pytest.mark.gpu


def _three_layer_round():
    wl = spec.small_round(n_agents=5)
    wl.shape.n_layers = 3
    return wl


_CASES = {"tiny_seg": lambda: spec.make("tiny_seg"), "small_round": lambda: spec.make("small_round"),
          "round_3_layers": _three_layer_round, "round_b256": lambda: spec.small_round(block_tokens=256),
          "tokendance": lambda: spec.make("tokendance")}


class Setup:
    def __init__(self, wl):
        self.wl = wl
        sh = wl.shape
        self.T = K.build_tables(sh, wl.agents)
        a = self.T.arrays
        self.a = a
        self.t = dedup.build_tables(sh.block_tokens, wl.agents)
        self.pool = wdev.Pool(wl, a["phys_agent"], a["phys_block"], a["phys_ntok"], a["n_dedup"])
        self.P = self.pool.capacity

    def dst(self, n, fill=0x7F7F):
        import torch
        sh = self.wl.shape
        shp = (sh.n_layers, n, sh.n_kv_heads, sh.block_tokens, sh.head_dim)
        k = torch.full(shp, fill, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        v = torch.full(shp, fill, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        return k, v

    def host_blocks(self, ids):
        """Pool bits of physical blocks ids: uint16 [L, len(ids), Hkv, B, d] (K, V)."""
        import torch
        idx = torch.from_numpy(np.asarray(ids, np.int64)).cuda()
        kh = self.pool.k.view(torch.int16).index_select(1, idx).cpu().numpy().view(np.uint16)
        vh = self.pool.v.view(torch.int16).index_select(1, idx).cpu().numpy().view(np.uint16)
        return kh, vh


def _dev32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.int32).reshape(-1)).cuda()


def _bits_of(x64):
    return (np.asarray(x64, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _host(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _agents_for(wl):
    n = wl.n_agents
    return list(range(n)) if n <= 12 else sorted({0, 1, n // 2, n - 1})


def _by_dst(lst):
    return lst[np.argsort(lst[:, 3], kind="stable")]


@pytest.mark.parametrize("name", list(_CASES))
def test_restore_matches_oracle(name):
    import torch
    wl = _CASES[name]()
    sh = wl.shape
    s = Setup(wl)
    tab = s.t
    h = sh.head_dim // 2
    for j in _agents_for(wl):
        lst = K.restore_list(s.T, j)
        m = len(lst)
        bd = _by_dst(lst)
        log(f"case {name}: restore agent {j}, {m} blocks, {int((lst[:, 1] != 0).sum())} shifted, "
            f"{len(set(lst[:, 0].tolist()))} sources")
        dk, dv = s.dst(m)
        K.kv_restore(sh, s.pool.k, s.pool.v, s.P, _dev32(lst), dk, dv, m)
        torch.cuda.synchronize()
        gk, gv = _host(dk), _host(dv)
        ids = sorted(set(int(x) for x in lst[:, 0]))
        where = {p: i for i, p in enumerate(ids)}
        kh, vh = s.host_blocks(ids)
        for layer in range(sh.n_layers):
            def stored(p, layer=layer):
                i, nt = where[p], int(tab["phys_ntok"][p])
                return (omir.bf16_bits_to_f64(kh[layer, i, :, :nt]).transpose(1, 0, 2),
                        omir.bf16_bits_to_f64(vh[layer, i, :, :nt]).transpose(1, 0, 2))
            Ke, Ve = omir.restore_blocks(tab, j, stored, sh.block_tokens, sh.rope_theta)
            ek, ev = _bits_of(Ke.transpose(0, 2, 1, 3)), _bits_of(Ve.transpose(0, 2, 1, 3))
            assert np.array_equal(gv[layer], ev)
            rot = np.repeat(bd[:, 1] != 0, sh.n_kv_heads * sh.block_tokens * sh.head_dim).reshape(ek.shape)
            assert np.array_equal(gk[layer][~rot], ek[~rot])
            if rot.any():
                gf = omir.bf16_bits_to_f64(gk[layer])
                ef = Ke.transpose(0, 2, 1, 3)
                pair = np.sqrt(ef[..., :h] ** 2 + ef[..., h:] ** 2)
                pair = np.concatenate([pair, pair], -1)
                ulp = np.abs(gk[layer].astype(np.int32) - ek.astype(np.int32)) <= 1
                near = np.abs(gf - ef) <= pair * 2.0 ** -20
                assert np.all((ulp | near)[rot])


@pytest.mark.parametrize("name", ["small_round", "round_3_layers", "round_b256", "tokendance"])
def test_restore_many_agents_in_one_call(name):
    """All agents (a repeat among them) restored by one call, entries grouped by
    source so that runs share their source read, are byte for byte the
    per-agent restores; a shuffled entry order gives the same bytes."""
    import torch
    wl = _CASES[name]()
    sh = wl.shape
    s = Setup(wl)
    agents = _agents_for(wl) + [_agents_for(wl)[0]]
    lst = K.restore_list(s.T, agents)
    n = len(lst)
    runs = int(np.sum(np.any(np.diff(lst[:, [0, 2]], axis=0) != 0, axis=1))) + 1
    log(f"case {name}: {len(agents)} agents, {n} entries, {runs} source runs")
    ak, av = s.dst(n)
    K.kv_restore(sh, s.pool.k, s.pool.v, s.P, _dev32(lst), ak, av, n)
    perm = np.random.default_rng(3).permutation(n)
    bk, bv = s.dst(n, fill=0x1111)
    K.kv_restore(sh, s.pool.k, s.pool.v, s.P, _dev32(lst[perm]), bk, bv, n)
    torch.cuda.synchronize()
    gk, gv = _host(ak), _host(av)
    assert np.array_equal(gk, _host(bk)) and np.array_equal(gv, _host(bv))
    off = 0
    for j in agents:
        one = K.restore_list(s.T, j)
        m = len(one)
        ok_, ov = s.dst(m)
        K.kv_restore(sh, s.pool.k, s.pool.v, s.P, _dev32(one), ok_, ov, m)
        torch.cuda.synchronize()
        assert np.array_equal(gk[:, off:off + m], _host(ok_)) and np.array_equal(gv[:, off:off + m], _host(ov))
        off += m
    assert off == n


@pytest.mark.parametrize("name", list(_CASES))
def test_fused_restore_equals_three_pass(name):
    """The unfused restore: gather the master of every logical block, overwrite
    the blocks that have a delta, re-rotate every K row by its block's shift."""
    import torch
    wl = _CASES[name]()
    sh = wl.shape
    s = Setup(wl)
    a = s.a
    for j in _agents_for(wl)[:3]:
        lst = K.restore_list(s.T, j)
        m = len(lst)
        nt = a["ntok"][j, :m]
        dst = np.arange(m)
        master = np.stack([a["block_table"][j, :m], np.zeros(m, np.int32), nt, dst], 1)
        dl = a["delta_table"][j, :m]
        delta = np.stack([np.where(dl >= 0, dl, -1), np.zeros(m, np.int32), nt, dst], 1)
        fk, fv = s.dst(m)
        K.kv_restore(sh, s.pool.k, s.pool.v, s.P, _dev32(lst), fk, fv, m)
        uk, uv = s.dst(m, fill=0x1234)
        K.kv_restore(sh, s.pool.k, s.pool.v, s.P, _dev32(master), uk, uv, m)
        K.kv_restore(sh, s.pool.k, s.pool.v, s.P, _dev32(delta), uk, uv, m)
        # third pass: one row per token (even agents) or per block of Hkv * B heads
        if j % 2 == 0:
            rows = uk.view(-1, 1, sh.head_dim)
            shift = np.tile(np.repeat(_by_dst(lst)[:, 1], sh.n_kv_heads * sh.block_tokens), sh.n_layers)
        else:
            rows = uk.view(-1, sh.n_kv_heads * sh.block_tokens, sh.head_dim)
            shift = np.tile(_by_dst(lst)[:, 1], sh.n_layers)
        K.kv_rerotate(rows, _dev32(shift), sh.rope_theta, out=rows)
        torch.cuda.synchronize()
        log(f"case {name}: agent {j}, {m} blocks, {int((dl >= 0).sum())} deltas")
        # the third pass also rotates the zeroed padding, which can turn +0 into
        # -0 (fused: padding is written as +0); every other bit must agree
        fkh, ukh = _host(fk), _host(uk)
        pad = np.zeros(fkh.shape, bool)
        for b in range(m):
            pad[:, b, :, int(nt[b]):] = True
        assert np.all(fkh[pad] == 0) and np.all((ukh[pad] & 0x7FFF) == 0)
        assert np.array_equal(fkh[~pad], ukh[~pad])
        assert np.array_equal(_host(fv), _host(uv))


def test_restore_skips_bad_entries():
    import torch
    wl = spec.make("tiny_seg")
    sh = wl.shape
    s = Setup(wl)
    lst = _by_dst(K.restore_list(s.T, 1)).copy()
    m = len(lst)
    lst[1, 0] = s.P           # id past the pool
    lst[2, 2] = sh.block_tokens + 1
    lst[3, 0] = -1
    lst[5, 3] = m             # destination past the buffer
    dk, dv = s.dst(m + 1, fill=0x5555)
    K.kv_restore(sh, s.pool.k, s.pool.v, s.P, _dev32(lst), dk, dv, m)
    torch.cuda.synchronize()
    gk, gv = _host(dk), _host(dv)
    for b in (1, 2, 3, 5, m):
        assert np.all(gk[:, b] == 0x5555) and np.all(gv[:, b] == 0x5555)
    for b in (0, 4, 6):
        assert not np.all(gk[:, b] == 0x5555)
    K.kv_restore(sh, s.pool.k, s.pool.v, s.P, None, None, None, 1)   # n = 0: nothing to do


def _gather_candidates(s, j):
    """Agent j's blocks in the master's stored frame (the restore with shift 0),
    destination b = logical block b."""
    lst = K.restore_list(s.T, j).copy()
    lst[:, 1] = 0
    ck, cv = s.dst(len(lst))
    K.kv_restore(s.wl.shape, s.pool.k, s.pool.v, s.P, _dev32(lst), ck, cv, len(lst))
    return lst, ck, cv


@pytest.mark.parametrize("name", ["small_round", "round_3_layers", "round_b256", "tokendance"])
def test_diff_recovers_delta_lists(name):
    """Each agent's blocks against their master: exactly the blocks that carry a
    delta differ (deltas hold other content), at threshold 0 and at a threshold
    below the smallest nonzero step of the contents; pairs in logical order and
    grouped by master."""
    import torch
    wl = _CASES[name]()
    sh = wl.shape
    s = Setup(wl)
    a = s.a
    for j in _agents_for(wl):
        lst, ck, cv = _gather_candidates(s, j)
        m = len(lst)
        pairs = np.stack([a["block_table"][j, :m], np.arange(m), a["ntok"][j, :m]], 1)
        want = (s.t["delta_table"][j, :m] >= 0).astype(np.int32)
        grouped = np.argsort(pairs[:, 0], kind="stable")
        for tau in (0.0, 1e-3):
            for order in (np.arange(m), grouped):
                flags = torch.full((m,), 7, dtype=torch.int32, device="cuda")
                K.kv_diff_blocks(sh, s.pool.k, s.pool.v, s.P, ck, cv, m, _dev32(pairs[order]), tau, flags)
                torch.cuda.synchronize()
                got = flags.cpu().numpy()
                log(f"case {name}: agent {j}, tau {tau}: {int(got.sum())} of {m} blocks differ")
                assert np.array_equal(got, want[order])


def test_diff_planted_against_oracle():
    import torch
    wl = _three_layer_round()
    sh = wl.shape
    s = Setup(wl)
    a = s.a
    j = 2
    lst, ck, cv = _gather_candidates(s, j)
    m = len(lst)
    nt = a["ntok"][j, :m].astype(np.int64)
    ckh, cvh = _host(ck).copy(), _host(cv).copy()
    g = np.random.default_rng(5)
    L, H, B, d = sh.n_layers, sh.n_kv_heads, sh.block_tokens, sh.head_dim
    planted = []
    for b in g.permutation(m)[: min(m, 40)]:
        b = int(b)
        kind = int(g.integers(0, 5))
        layer, hh, e = int(g.integers(0, L)), int(g.integers(0, H)), int(g.integers(0, d))
        t = int(g.integers(0, nt[b]))
        buf = ckh if g.random() < 0.5 else cvh
        if kind == 0:
            buf[layer, b, hh, t, e] ^= 1                          # lowest mantissa bit
        elif kind == 1 and nt[b] < B:
            buf[layer, b, hh, int(g.integers(nt[b], B)), e] ^= 0x4000   # padding only
        elif kind == 2:
            buf[layer, b, hh, t, e] = 0x7FC0                      # NaN
        elif kind == 3:
            buf[L - 1, b, H - 1, nt[b] - 1, d - 1] ^= 0x0100      # last valid value of the last layer
        planted.append((b, kind))
    log(f"planted {len(planted)} changes over {m} candidate blocks")
    ck2 = torch.from_numpy(ckh.view(np.int16)).cuda()
    cv2 = torch.from_numpy(cvh.view(np.int16)).cuda()
    pairs = np.stack([a["block_table"][j, :m], np.arange(m), nt], 1)
    mk, mv = s.host_blocks(pairs[:, 0])
    mk, mv = mk.transpose(1, 0, 2, 3, 4), mv.transpose(1, 0, 2, 3, 4)
    grouped = np.argsort(pairs[:, 0], kind="stable")
    for tau in (0.0, 1e-2, 0.5):
        want = omir.diff_flags(mk, mv, ckh.transpose(1, 0, 2, 3, 4), cvh.transpose(1, 0, 2, 3, 4), nt, tau)
        for order in (np.arange(m), grouped):
            flags = torch.zeros(m, dtype=torch.int32, device="cuda")
            K.kv_diff_blocks(sh, s.pool.k, s.pool.v, s.P, ck2, cv2, m, _dev32(pairs[order]), tau, flags)
            torch.cuda.synchronize()
            got = flags.cpu().numpy()
            log(f"tau {tau}: {int(got.sum())} flagged")
            assert np.array_equal(got, want[order])
    bad = pairs.copy()
    bad[0, 0], bad[1, 1], bad[2, 2] = s.P, m, B + 1
    flags = torch.zeros(m, dtype=torch.int32, device="cuda")
    K.kv_diff_blocks(sh, s.pool.k, s.pool.v, s.P, ck2, cv2, m, _dev32(bad), 0.0, flags)
    torch.cuda.synchronize()
    got = flags.cpu().numpy()
    assert list(got[:3]) == [-1, -1, -1]
