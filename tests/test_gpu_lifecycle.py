"""Block lifecycle on the GPU through the C ABI: kv_append's block copies and
token writes byte for byte against what the oracle replay prescribes, and decode
attention after rounds of appends (with copy-on-write) and destroys against the
oracle's dense recomputation from its content model."""
import numpy as np
import pytest

from oracle import attention as oatt
from oracle import dedup
from oracle import lifecycle as olc
from oracle import rope
from shared_paged_kv_amd import _lib as K
from workload import device as wdev
from workload import rng, spec

from .gpu_util import log
from .tolerances import ATOL, gate

pytestmark = pytest.mark.gpu


def _bits(x64):
    """bf16-valued float64 array -> uint16 bits."""
    return (np.asarray(x64, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _new_rows(g, sh, n):
    """Seeded new-token K and V: [n_layers, n, Hkv, d] bf16-valued float64."""
    shp = (sh.n_layers, n, sh.n_kv_heads, sh.head_dim)
    return olc.bf16_round(g.standard_normal(shp)), olc.bf16_round(g.standard_normal(shp))


def _upload_rows(kr, vr):
    import torch
    k = torch.from_numpy(_bits(kr).view(np.int16)).cuda().view(torch.bfloat16)
    v = torch.from_numpy(_bits(vr).view(np.int16)).cuda().view(torch.bfloat16)
    return k, v


def _ops_dev(cp, wr):
    import torch
    c = torch.from_numpy(np.ascontiguousarray(cp, np.int32).reshape(-1)).cuda() if len(cp) else None
    w = torch.from_numpy(np.ascontiguousarray(wr, np.int32).reshape(-1)).cuda() if len(wr) else None
    return c, w


class Setup:
    def __init__(self, wl, extra):
        self.wl = wl
        sh = wl.shape
        self.T = K.build_tables(sh, wl.agents)
        self.t = dedup.build_tables(sh.block_tokens, wl.agents)
        a = self.T.arrays
        self.cap = self.T.n_phys + extra
        self.pool = wdev.Pool(wl, a["phys_agent"], a["phys_block"], a["phys_ntok"], a["n_dedup"], capacity=self.cap)
        self.bp = K.BlockPool(self.T, sh, self.cap)

    def append(self, sel, kr, vr, replays=()):
        """Library append + kv_append; the same append on every oracle replay
        (replays: list of (PoolReplay, layer, kv heads modelled))."""
        import torch
        cp, wr = self.bp.append(sel)
        for r, layer, kvh in replays:
            oc, ow = r.append(sel, kr[layer][:, kvh], vr[layer][:, kvh], self.wl.shape.rope_theta)
            assert [tuple(x) for x in cp.tolist()] == oc and [tuple(x) for x in wr.tolist()] == ow
        c, w = _ops_dev(cp, wr)
        kd, vd = _upload_rows(kr, vr)
        K.kv_append(self.wl.shape, self.pool.k, self.pool.v, self.cap, c, w, kd, vd, len(sel))
        torch.cuda.synchronize()
        return cp, wr


def _stored_fn(wl, t, layer, kvh):
    store = oatt._Store(wl, layer)

    def stored(p):
        j, b = int(t["phys_agent"][p]), int(t["phys_block"][p])
        seed = wl.blk_delta_seed[j][b] if p >= t["n_dedup"] else wl.blk_seed[j][b]
        nt = int(t["phys_ntok"][p])
        Kb = np.stack([store.get(seed, nt, g)[0] for g in kvh], 1)
        Vb = np.stack([store.get(seed, nt, g)[1] for g in kvh], 1)
        return Kb, Vb
    return stored


def _attend_sel(qf, Kd, Vd, heads, kvh, grp, scale):
    """Attention of q heads `heads` over K, V [L, len(kvh), d] holding kv heads kvh."""
    out = np.zeros((len(heads), qf.shape[-1]))
    for i, h in enumerate(heads):
        g = kvh.index(h // grp)
        s = (Kd[:, g, :] @ qf[h]) * scale
        p = np.exp(s - s.max())
        out[i] = (p @ Vd[:, g, :]) / p.sum()
    return out


_APPEND_CASES = {"tiny_seg": lambda: spec.make("tiny_seg"), "small_round": lambda: spec.make("small_round"),
                 "round_b256": lambda: spec.small_round(block_tokens=256)}


@pytest.mark.parametrize("name", list(_APPEND_CASES))
def test_kv_append_bytes_match_replay(name):
    """After each append: copied blocks are the sources' bytes (every layer,
    head and slot), written slots hold V as given and K rotated by -shift
    (within 1 bf16 ulp of the float64 rotation; bit-exact where shift is 0),
    and nothing else changed."""
    import torch
    wl = _APPEND_CASES[name]()
    sh = wl.shape
    s = Setup(wl, 96)
    g = np.random.default_rng(21)
    log(f"case {name}: kv_append bytes, capacity {s.cap}")
    for rnd in range(3):
        kh = s.pool.k.view(torch.int16).cpu().numpy().view(np.uint16).copy()
        vh = s.pool.v.view(torch.int16).cpu().numpy().view(np.uint16).copy()
        sel = [int(x) for x in g.integers(0, wl.n_agents, size=wl.n_agents + 3)]
        kr, vr = _new_rows(g, sh, len(sel))
        cp, wr = s.append(sel, kr, vr)
        log(f"  round {rnd}: {len(cp)} copies, {len(wr)} writes")
        ek, ev = kh.copy(), vh.copy()
        for src, dst in cp.tolist():
            ek[:, dst] = ek[:, src]
            ev[:, dst] = ev[:, src]
        tol = np.zeros_like(ek, dtype=bool)
        for p, slot, row, shift in wr.tolist():
            for layer in range(sh.n_layers):
                kx = kr[layer, row]
                if shift:
                    kx = olc.bf16_round(rope.rotate(kx, -shift, sh.rope_theta))
                    tol[layer, p, :, slot] = True
                ek[layer, p, :, slot] = _bits(kx)
                ev[layer, p, :, slot] = _bits(vr[layer, row])
        gk = s.pool.k.view(torch.int16).cpu().numpy().view(np.uint16)
        gv = s.pool.v.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(gv, ev)
        assert np.array_equal(gk[~tol], ek[~tol])
        d = np.abs(gk[tol].astype(np.int32) - ek[tol].astype(np.int32))
        assert d.size == 0 or d.max() <= 1
        log(f"  rotated K slots: {d.size} values, {int((d > 0).sum())} differ by 1 ulp")


def _three_layer_round():
    wl = spec.small_round(n_agents=5)
    wl.shape.n_layers = 3
    return wl


_DECODE_CASES = {"tiny_seg": lambda: spec.make("tiny_seg"), "small_round": lambda: spec.make("small_round"),
                 "tiny": lambda: spec.make("tiny"), "round_3_layers": _three_layer_round,
                 "round_b256": lambda: spec.small_round(block_tokens=256)}


@pytest.mark.parametrize("name", list(_DECODE_CASES))
def test_decode_after_appends_and_destroy(name):
    """Rounds of appends (copy-on-write where blocks are shared), a destroyed
    agent, then the decode through the pool's snapshot plan against attention
    over the oracle's dense contexts (first and last layer: the pool's layer
    stride is its capacity)."""
    import torch
    wl = _DECODE_CASES[name]()
    sh = wl.shape
    s = Setup(wl, 160)
    kvh = list(range(sh.n_kv_heads))
    layers = sorted({0, sh.n_layers - 1})
    replays = [(olc.PoolReplay(s.t, sh.block_tokens, s.cap), layer, kvh) for layer in layers]
    for r, layer, _ in replays:
        r.model_contents(_stored_fn(wl, s.t, layer, kvh))
    g = np.random.default_rng(33)
    dead = 1 % wl.n_agents
    n_cp = 0
    for rnd in range(5):
        live = [j for j in range(wl.n_agents) if replays[0][0].alive[j] == "live"]
        sel = [int(x) for x in g.choice(live, size=2 * len(live))]
        kr, vr = _new_rows(g, sh, len(sel))
        cp, _ = s.append(sel, kr, vr, replays)
        n_cp += len(cp)
        if rnd == 2:
            s.bp.destroy(dead)
            for r, _, _ in replays:
                r.destroy(dead)
    log(f"case {name}: {n_cp} copy-on-write copies over 5 rounds, agent {dead} destroyed")
    S = s.bp.tables()
    au = s.bp.audit()
    assert au["n_leaked"] == 0 and au["n_mismatched"] == 0
    plan = K.DevicePlan(S)
    ws = torch.empty(max(1, K.workspace_bytes(sh, plan)), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.n_agents, sh.n_q_heads, sh.head_dim), dtype=torch.float32, device="cuda")
    grp = sh.n_q_heads // sh.n_kv_heads
    scale = 1.0 / np.sqrt(sh.head_dim)
    for r, layer, _ in replays:
        q = wdev.fill_q(wl, layer)
        K.paged_decode_attn(sh, plan, q, s.pool.k, s.pool.v, out, ws, layer=layer)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        qf = rng.bf16_bits_to_f32(spec.q_bits(wl, layer)).astype(np.float64)
        worst = 0.0
        for j in range(wl.n_agents):
            if j == dead:
                assert np.all(got[j] == 0.0)
                continue
            Kd, Vd = r.dense(j, sh.rope_theta)
            ref = _attend_sel(qf[j], Kd, Vd, list(range(sh.n_q_heads)), kvh, grp, scale)
            err = float(np.abs(got[j] - ref).max())
            worst = max(worst, err)
            assert err <= ATOL and err <= gate(ref, Kd.shape[0]), (j, err)
        log(f"  layer {layer}: max-abs {worst:.3e} over the live agents")


def test_tokendance_round_append_copy_on_write():
    """TokenDance round: every agent ends with the same shared segment, read at
    64 different shifts; one append each copies its last block for every sharer
    but the last and writes each token in its copy's frame.  Decode of sampled agents and heads after two
    appends matches the oracle."""
    import torch
    # the seed-0 round's last segment fills its last block; trim it by 5 tokens
    # for every agent so that the block they share has room for the append
    base = spec.make("tokendance")
    agents_in = []
    for ag in base.agents:
        sp = list(ag.spans)
        sp[-1] = spec.Span(sp[-1].tier, sp[-1].group, sp[-1].kind, sp[-1].tokens[:-5])
        agents_in.append(spec.Agent(sp, ag.delta_blocks.copy()))
    wl = spec.describe(spec.Workload("tokendance_trim5", base.seed, base.shape, agents_in))
    sh = wl.shape
    s = Setup(wl, 512)
    last = s.t["n_blocks"] - 1
    n_share = sum(1 for j in range(wl.n_agents) if s.t["delta_table"][j, last[j]] < 0)
    agents, kvh = [0, 21, 63], [0, 5]
    grp = sh.n_q_heads // sh.n_kv_heads
    heads = [h for h in range(sh.n_q_heads) if h // grp in kvh]
    r = olc.PoolReplay(s.t, sh.block_tokens, s.cap)
    # model the contents the sampled agents read (others' writes are bookkept only)
    stored = _stored_fn(wl, s.t, 0, kvh)
    for j in agents:
        for e in r.entries[j]:
            p = r._eff(e)
            if p not in r.content:
                r.content[p] = stored(p)
    g = np.random.default_rng(44)
    log("case tokendance: two appends for all 64 agents")
    for rnd in range(2):
        sel = list(range(wl.n_agents))
        kr, vr = _new_rows(g, sh, len(sel))
        cp, wr = s.append(sel, kr, vr, [(r, 0, kvh)])
        log(f"  round {rnd}: {len(cp)} copies, {int((wr[:, 3] != 0).sum())} writes with a shift")
        if rnd == 0:
            # all but the last sharer copy; agents with a delta there write into it
            assert len(cp) == n_share - 1 and n_share > 32
    S = s.bp.tables()
    plan = K.DevicePlan(S)
    ws = torch.empty(max(1, K.workspace_bytes(sh, plan)), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.n_agents, sh.n_q_heads, sh.head_dim), dtype=torch.float32, device="cuda")
    q = wdev.fill_q(wl, 0)
    K.paged_decode_attn(sh, plan, q, s.pool.k, s.pool.v, out, ws, layer=0)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    qf = rng.bf16_bits_to_f32(spec.q_bits(wl, 0)).astype(np.float64)
    scale = 1.0 / np.sqrt(sh.head_dim)
    for j in agents:
        Kd, Vd = r.dense(j, sh.rope_theta)
        ref = _attend_sel(qf[j], Kd, Vd, heads, kvh, grp, scale)
        err = float(np.abs(got[j, heads] - ref).max())
        log(f"  agent {j}: {Kd.shape[0]} tokens, max-abs {err:.3e}")
        assert err <= ATOL and err <= gate(ref, Kd.shape[0])
