"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Attention output: max-abs <= ATOL (2e-3) and <= the tighter internal gate;
everything integer is compared bit for bit elsewhere (test_tables_cpu.py)."""
import math

import numpy as np
import pytest

from oracle import attention, rope
from shared_paged_kv_amd import _lib as K
from workload import rng, spec

from .gpu_util import Case, log
from .tolerances import ATOL, gate

pytestmark = pytest.mark.gpu


def _cmp(name, got, ref, L, agents=None, heads=None):
    if agents is not None:
        got = got[agents]
    if heads is not None:
        got, ref = got[:, heads], ref[:, heads]
    err = float(np.abs(got - ref).max())
    g = gate(ref, L)
    log(f"{name}: max-abs {err:.3e}  gate {g:.3e}  rms(ref) {np.sqrt(np.mean(ref**2)):.3e}")
    assert np.isfinite(got).all()
    assert err <= ATOL
    assert err <= g


def test_generator_device_matches_host():
    """The device filler reproduces the host generator bit for bit (bf16 pool,
    Q4 codes and params, queries), padding slots included."""
    import torch
    for name in ["tiny_seg", "tiny_q4"]:
        wl = spec.make(name)
        c = Case(wl)
        a = c.T.arrays
        for p in [0, a["n_phys"] // 2, a["n_phys"] - 1]:
            j, b = int(a["phys_agent"][p]), int(a["phys_block"][p])
            seed = wl.blk_delta_seed[j][b] if p >= a["n_dedup"] else wl.blk_seed[j][b]
            nt = int(a["phys_ntok"][p])
            kb = spec.block_kv_bits(seed, wl.shape, 0, nt, rng.SEL_K)
            vb = spec.block_kv_bits(seed, wl.shape, 0, nt, rng.SEL_V)
            if wl.shape.kv_dtype == spec.BF16:
                assert np.array_equal(c.pool.k[0, p].view(torch.int16).cpu().numpy().view(np.uint16), kb)
                assert np.array_equal(c.pool.v[0, p].view(torch.int16).cpu().numpy().view(np.uint16), vb)
            else:
                for t, tp, bits in ((c.pool.k, c.pool.kp, kb), (c.pool.v, c.pool.vp, vb)):
                    codes, params = rng.q4_encode(bits)
                    assert np.array_equal(t[0, p].cpu().numpy(), codes)
                    assert np.array_equal(tp[0, p].view(torch.int16).cpu().numpy().view(np.uint16),
                                          params.view(np.uint16))
        q = c.q(0).view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(q, spec.q_bits(wl, 0))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rerotate_matches_oracle(dtype):
    import torch
    from shared_paged_kv_amd import kv_rerotate
    r = np.random.default_rng(0)
    R, H, d, base = 300, 3, 128, 1e6
    bits = rng.bf16_tile((1, 2, 3, 4), 0, 0, (R, H, d))
    xf = rng.bf16_bits_to_f32(bits)
    shift = r.integers(-45000, 45000, size=R).astype(np.int32)
    shift[:5] = 0
    x = torch.from_numpy(xf).cuda().to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    s = torch.from_numpy(shift).cuda()
    y = kv_rerotate(x, s, base).float().cpu().numpy().astype(np.float64)
    ref = rope.rotate(xf.astype(np.float64), shift[:, None], base)
    if dtype == "bf16":
        # within one bf16 ulp of the exact value
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert (np.abs(y - ref) <= ulp + 1e-30).all()
    else:
        assert np.abs(y - ref).max() < 2e-5
    # zero shift is the identity, bit for bit
    assert np.array_equal(y[:5], xf[:5].astype(np.float64))
    # in place
    x2 = x.clone()
    kv_rerotate(x2, s, base, out=x2)
    assert torch.equal(x2, kv_rerotate(x, s, base))


@pytest.mark.parametrize("d", [16, 48, 64, 128, 256, 512])
@pytest.mark.parametrize("dts", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16"), ("f32", "f32")])
def test_rerotate_vector_path_equals_scalar_path(d, dts):
    """Buffers 16-byte aligned with head_dim a multiple of 16 take the vector
    kernel; the same data one element off alignment takes the per-pair kernel.
    Both form cos/sin by the same float64 steps and round the same way, so the
    outputs agree bit for bit (and with the oracle's rotation within a bf16 ulp
    or 2e-5 in float32)."""
    import torch
    from shared_paged_kv_amd import kv_rerotate
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    r = np.random.default_rng(d)
    R, H, base = 77, 5, 1e4
    xf = r.standard_normal((R, H, d)).astype(np.float32)
    shift = r.integers(-30000, 30000, size=R).astype(np.int32)
    s = torch.from_numpy(shift).cuda()
    x = torch.from_numpy(xf).cuda().to(tdt[dts[0]])
    n = R * H * d
    xs = torch.zeros(n + 8, dtype=tdt[dts[0]], device="cuda")
    xs[1:1 + n] = x.reshape(-1)
    ys = torch.zeros(n + 8, dtype=tdt[dts[1]], device="cuda")
    xm, ym = xs[1:1 + n].view(R, H, d), ys[1:1 + n].view(R, H, d)
    assert xm.data_ptr() % 16 and x.data_ptr() % 16 == 0
    yv = kv_rerotate(x, s, base, out_dtype=tdt[dts[1]])
    kv_rerotate(xm, s, base, out=ym)
    assert torch.equal(yv, ym)
    xd = x.float().cpu().numpy().astype(np.float64)
    ref = rope.rotate(xd, shift[:, None], base)
    y = yv.float().cpu().numpy().astype(np.float64)
    if dts[1] == "bf16":
        # one bf16 ulp of the exact value, plus the float32 rotation's own error
        # (a few 2^-24 of the pair's norm), which matters where the pair cancels
        h = d // 2
        pair = np.sqrt(xd[..., :h] ** 2 + xd[..., h:] ** 2)
        pair = np.concatenate([pair, pair], -1)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert (np.abs(y - ref) <= ulp + pair * 2.0 ** -20).all()
    else:
        assert np.abs(y - ref).max() < 2e-5 * max(1.0, np.abs(ref).max())


def test_rerotate_composes():
    """R(b) R(a)^-1 x == R(b - a) x on the device (float32 path)."""
    import torch
    from shared_paged_kv_amd import kv_rerotate
    r = np.random.default_rng(1)
    x = torch.from_numpy(r.standard_normal((64, 2, 64)).astype(np.float32)).cuda()
    a = torch.from_numpy(r.integers(0, 4000, 64).astype(np.int32)).cuda()
    b = torch.from_numpy(r.integers(0, 4000, 64).astype(np.int32)).cuda()
    two = kv_rerotate(kv_rerotate(x, -a, 1e4), b, 1e4)
    one = kv_rerotate(x, b - a, 1e4)
    assert (two - one).abs().max().item() < 1e-4


@pytest.mark.parametrize("name", ["tiny", "tiny_seg", "tiny_q4", "small_round"])
def test_decode_small(name):
    wl = spec.make(name)
    log("case", name)
    c = Case(wl)
    got = c.run(0)
    ref = attention.decode(wl, 0)
    _cmp(name, got, ref, max(wl.context_len(j) for j in range(wl.n_agents)))


def test_decode_q4_block256_small():
    wl = spec.tiny_q4(block_tokens=256)
    c = Case(wl)
    got = c.run(0)
    ref = attention.decode(wl, 0)
    _cmp("tiny_q4_b256", got, ref, max(wl.context_len(j) for j in range(wl.n_agents)))


@pytest.mark.parametrize("hq,hkv", [(10, 2), (4, 4)])
def test_decode_bf16_block256(hq, hkv):
    """bf16 pools with 256-token blocks: 16 tiles per block, partial blocks,
    shared segments read by many rows (GQA 5) or one row per kv head (MHA)."""
    wl = spec.small_round(hq=hq, hkv=hkv, block_tokens=256)
    c = Case(wl)
    got = c.run(0)
    ref = attention.decode(wl, 0)
    _cmp(f"small_round_b256_{hq}x{hkv}", got, ref, max(wl.context_len(j) for j in range(wl.n_agents)))


def test_decode_multi_layer_tiny_round():
    """Layer indexing: a 3-layer round, each layer checked against the oracle."""
    wl = spec.small_round(n_agents=5)
    wl.shape.n_layers = 3
    c = Case(wl)
    for layer in range(3):
        _cmp(f"layer{layer}", c.run(layer), attention.decode(wl, layer), 1200)


def test_edge_cases():
    """Empty agent (zero output), one-token spans, exact block multiples, a
    segment repeated inside one agent, and a delta on a repeated segment."""
    P, G, S = spec.PRIVATE, spec.GROUP, spec.SEGMENT
    g = np.random.default_rng(3)
    tk = lambda n: g.integers(1, 1 << 30, n).astype(np.int32)
    seg = tk(40)
    agents = [
        spec.Agent([]),
        spec.Agent([spec.Span(P, 0, spec.PREFIX, tk(1))]),
        spec.Agent([spec.Span(spec.GLOBAL, 0, spec.PREFIX, tk(32)), spec.Span(P, 0, spec.PREFIX, tk(16))]),
        spec.Agent([spec.Span(G, 2, S, seg), spec.Span(P, 0, spec.PREFIX, tk(3)), spec.Span(G, 2, S, seg)]),
        spec.Agent([spec.Span(P, 0, spec.PREFIX, tk(7)), spec.Span(G, 2, S, seg)], np.array([1, 3], np.int32)),
    ]
    wl = spec.describe(spec.Workload("edge", 0, spec.Shape(1, 4, 2, 128, 16, spec.BF16, 1e4), agents))
    c = Case(wl)
    got = c.run(0)
    ref = attention.decode(wl, 0)
    assert not got[0].any()
    _cmp("edge", got, ref, 100)


@pytest.mark.parametrize("n_agents", [0, 3])
def test_decode_all_agents_empty(n_agents):
    """No cached token anywhere: no physical block and no work item, so the pools
    are empty (NULL) tensors.  With agents every output is zero (the combine runs
    alone); without agents nothing is enqueued."""
    wl = spec.describe(spec.Workload("empty", 0, spec.Shape(1, 8, 2, 128, 16, spec.BF16, 1e4),
                                     [spec.Agent([]) for _ in range(n_agents)]))
    c = Case(wl)
    assert c.T.arrays["n_phys"] == 0 and c.T.arrays["items"].shape[0] == 0
    c.out.fill_(7.0)
    got = c.run(0)
    assert got.shape == (n_agents, 8, 128) and not got.any()


def test_decode_large_shift():
    """A shared segment read about 100k positions after its stored frame (and
    37 after it by a third agent): the tile pass rotates that consumer's query by
    R(-100000), from the plan's float32 cos and sin of float64 angles of up to
    1e5 rad, and the outputs stay within ATOL and the gate of the oracle, which
    rotates the stored keys in float64."""
    g = np.random.default_rng(77)
    tk = lambda m: g.integers(1, 1 << 30, m).astype(np.int32)
    seg = tk(200)
    agents = [spec.Agent([spec.Span(spec.GROUP, 5, spec.SEGMENT, seg)]),
              spec.Agent([spec.Span(spec.PRIVATE, 0, spec.PREFIX, tk(100000)), spec.Span(spec.GROUP, 5, spec.SEGMENT, seg)]),
              spec.Agent([spec.Span(spec.PRIVATE, 0, spec.PREFIX, tk(37)), spec.Span(spec.GROUP, 5, spec.SEGMENT, seg)])]
    wl = spec.describe(spec.Workload("large_shift", 77, spec.Shape(1, 4, 2, 64, 16, spec.BF16, 1e4), agents))
    log("case large_shift")
    c = Case(wl)
    a = c.T.arrays
    assert a["shift"].max() == 100000 and 37 in a["shift"][2]
    got = c.run(0)
    ref = attention.decode(wl, 0)
    _cmp_agents("large_shift", got, ref, wl, list(range(wl.n_agents)))


def test_needle_in_shifted_segment():
    """A key planted in a shifted segment block: stored as R(-shift) k so that the
    agent reads k, whose score 40 dominates; the output must be that token's V.
    A wrong rotation direction scatters the score and fails."""
    import torch
    wl = spec.make("small_round")
    c = Case(wl)
    a = c.T.arrays
    j, h = 7, 3
    g = h // (wl.shape.n_q_heads // wl.shape.n_kv_heads)
    # a segment block of agent j with a non-zero shift and no delta
    bs = [b for b in spec.segment_block_ids(wl, j) if a["delta_table"][j, b] < 0 and a["shift"][j, b] != 0]
    b = bs[len(bs) // 2]
    p, shift, t = int(a["block_table"][j, b]), int(a["shift"][j, b]), 2
    q = c.q(0)
    qv = q[j, h].float().cpu().numpy().astype(np.float64)
    d = wl.shape.head_dim
    k = 40 * math.sqrt(d) * qv / (qv @ qv)
    stored = rope.rotate(k, -shift, wl.shape.rope_theta)
    c.pool.k[0, p, g, t] = torch.from_numpy(stored.astype(np.float32)).to(torch.bfloat16).cuda()
    got = c.run(0, q=q)
    vt = c.pool.v[0, p, g, t].float().cpu().numpy()
    # the planted key is rounded to bf16, so its score is 40 up to ~0.3
    assert np.abs(got[j, h] - vt).max() < 1e-3


def _cmp_agents(name, got, ref, wl, agents):
    """Every (agent, q head, dim) output against the oracle's: max-abs within ATOL
    and, per agent, within the internal gate for that agent's context length."""
    worst = (0.0, None)
    for i, j in enumerate(agents):
        err = float(np.abs(got[i] - ref[i]).max())
        assert np.isfinite(got[i]).all(), f"{name}: agent {j} has non-finite outputs"
        g = gate(ref[i], wl.context_len(j))
        assert err <= ATOL and err <= g, f"{name}: agent {j} max-abs {err:.3e} (gate {g:.3e})"
        worst = max(worst, (err / g, j))
    err = float(np.abs(got - ref).max())
    log(f"{name}: {len(agents)} agents x {got.shape[1]} heads x {got.shape[2]} dims, max-abs {err:.3e}, "
        f"worst error / gate {worst[0]:.3f} (agent {worst[1]})")


@pytest.mark.parametrize("name", ["inms", "tokendance", "q4"])
def test_decode_full_size_all_outputs(name):
    """Full-size configs, launched exactly as the bench launches them; every
    output of every agent and q head against the oracle's (stored by
    tests/golden/make_fullsize.py, which runs only the oracle)."""
    from tests.golden import make_fullsize as golden
    wl = spec.make(name)
    ref, agents, layers = golden.load(name, wl)
    assert layers == [0] and agents == list(range(wl.n_agents))
    log("case", name, "all", len(agents), "agents")
    c = Case(wl)
    got = c.run(0)
    _cmp_agents(name, got, ref[0], wl, agents)


def test_phases_equal_single_call():
    """Query prep, tile pass and combine issued apart (1, 2, 4) give bit-for-bit
    the single call's output, on a config with shifted consumers."""
    import torch
    from shared_paged_kv_amd import _lib as K
    wl = spec.make("small_round")
    c = Case(wl)
    q = c.q(0)
    one = c.run(0, q=q)
    c.out.zero_()
    for ph in (K.PHASE_QPREP, K.PHASE_TILES, K.PHASE_COMBINE):
        K.paged_decode_attn_phases(wl.shape, c.plan, q, c.pool.k, c.pool.v, c.out, c.ws, ph)
    torch.cuda.synchronize()
    assert np.array_equal(c.out.cpu().numpy().astype(np.float64), one)


def test_decode_scale_full_size():
    """The scale config at full size: 250 agents, all 48 layers resident
    (~232 GB of deduplicated bf16 KV), every layer launched as in a decode step;
    at the first and last layer every q head of 32 agents -- both ends, one in the middle and three
    from each of the ten consumer groups the shared segments are split into --
    against the oracle's stored outputs."""
    import gc
    import torch
    from tests.golden import make_fullsize as golden
    gc.collect()
    torch.cuda.empty_cache()
    wl = spec.make("scale")
    ref, agents, layers = golden.load("scale", wl)
    log("case scale: building tables and filling 48 layers")
    c = Case(wl)
    outs = {}
    for layer in range(wl.shape.n_layers):
        got = c.run(layer)
        assert np.isfinite(got).all()
        if layer in layers:
            outs[layer] = got[agents]
    log("scale: 48 layers done")
    for li, layer in enumerate(layers):
        _cmp_agents(f"scale layer {layer}", outs[layer], ref[li], wl, agents)
    del c
    gc.collect()
    torch.cuda.empty_cache()


def _private_twin(wl):
    """The same agents with every span PRIVATE (nothing shared, no deltas)."""
    agents = [spec.Agent([spec.Span(spec.PRIVATE, 0, sp.kind, sp.tokens) for sp in ag.spans]) for ag in wl.agents]
    return spec.Workload(wl.name + "_private", wl.seed, spec.Shape(**vars(wl.shape)), agents)


@pytest.mark.parametrize("name", ["tiny", "tiny_seg", "small_round"])
def test_sharing_invariance_on_device(name):
    """Outputs do not depend on sharing (TokenDance write-up, evaluation): the
    library's dedup tables over the shared pool against all-PRIVATE tables whose
    pool holds, per agent and logical block, exactly what that agent reads there
    (delta applied, key moved to the agent's own position by the oracle's RoPE,
    rounded to bf16)."""
    import torch
    from shared_paged_kv_amd import _lib as K
    from oracle import rope as orope
    wl = spec.make(name)
    shared = Case(wl)
    q = shared.q(0)
    out_shared = shared.run(0, q=q)
    tw = _private_twin(wl)
    T = K.build_tables(tw.shape, tw.agents)
    a = T.arrays
    assert a["n_dedup"] == sum(wl.n_blocks(j) for j in range(wl.n_agents))
    sh = wl.shape
    k = torch.empty((1, a["n_phys"], sh.n_kv_heads, sh.block_tokens, sh.head_dim), dtype=torch.bfloat16)
    v = torch.empty_like(k)
    dense = {}  # agent -> list of (K, V) float64 blocks as stored in the twin's pool
    for p in range(a["n_phys"]):
        j, b = int(a["phys_agent"][p]), int(a["phys_block"][p])
        seed, nt = spec.logical_seed(wl, j, b), int(wl.blk_ntok[j][b])
        shift = int(wl.blk_pos0[j][b]) - int(wl.blk_frame[j][b])
        kb = rng.bf16_bits_to_f32(spec.block_kv_bits(seed, sh, 0, nt, rng.SEL_K)).astype(np.float64)
        vb = rng.bf16_bits_to_f32(spec.block_kv_bits(seed, sh, 0, nt, rng.SEL_V))
        kr = orope.rotate(np.nan_to_num(kb), shift, sh.rope_theta) if shift else kb
        kr[:, nt:, :] = np.nan
        k[0, p] = torch.from_numpy(kr.astype(np.float32)).to(torch.bfloat16)
        v[0, p] = torch.from_numpy(vb).to(torch.bfloat16)
        kst = k[0, p, :, :nt].float().numpy().astype(np.float64).transpose(1, 0, 2)
        dense.setdefault(j, []).append((b, kst, vb[:, :nt].astype(np.float64).transpose(1, 0, 2)))
    plan = K.DevicePlan(T)
    ws = torch.empty(max(1, K.workspace_bytes(tw.shape, plan)), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(shared.out)
    K.paged_decode_attn(tw.shape, plan, q, k.cuda(), v.cuda(), out, ws)
    torch.cuda.synchronize()
    out_private = out.cpu().numpy().astype(np.float64)
    ref = attention.decode(wl, 0)
    L = max(wl.context_len(j) for j in range(wl.n_agents))
    _cmp(name + " shared", out_shared, ref, L)
    # the twin against the exact attention over what its pool stores
    qf = rng.bf16_bits_to_f32(spec.q_bits(wl, 0)).astype(np.float64)
    ref_twin = np.zeros_like(ref)
    for j, blocks in dense.items():
        blocks.sort(key=lambda x: x[0])
        Kd = np.concatenate([kb for _, kb, _ in blocks])
        Vd = np.concatenate([vb for _, _, vb in blocks])
        ref_twin[j] = attention.attend(qf[j], Kd, Vd, 1 / math.sqrt(sh.head_dim))
    _cmp(name + " private twin", out_private, ref_twin, L)
    # with and without sharing: equal up to the bf16 rounding of moved keys
    d = float(np.abs(out_shared - out_private).max())
    log(f"{name}: shared vs private twin {d:.3e}")
    assert d <= ATOL
    if name == "tiny":  # no shifts: no key is moved, only summation orders differ
        assert d < 1e-6


@pytest.mark.parametrize("n,prefix,tail", [(4, 128, 70), (6, 1200, 900)])
def test_agent_order_invariance(n, prefix, tail):
    """Reversing the agents relabels every physical block and changes the plan;
    each agent's output stays the same.  Each agent's tail is its own GROUP
    (not PRIVATE), so a block's content does not depend on the agent's index."""
    import torch
    g = np.random.default_rng(9)
    pre = g.integers(1, 1 << 30, prefix).astype(np.int32)
    agents = [spec.Agent([spec.Span(spec.GLOBAL, 0, spec.PREFIX, pre),
                          spec.Span(spec.GROUP, 100 + j, spec.PREFIX, g.integers(1, 1 << 30, tail + 7 * j).astype(np.int32))])
              for j in range(n)]
    shape = spec.Shape(1, 8, 2, 128, 16, spec.BF16, 1e4)
    wl = spec.describe(spec.Workload("order", 0, shape, agents))
    rev = spec.describe(spec.Workload("order", 0, spec.Shape(**vars(shape)), agents[::-1]))
    c, cr = Case(wl), Case(rev)
    q = c.q(0)
    got = c.run(0, q=q)
    got_rev = cr.run(0, q=torch.flip(q, dims=[0]).contiguous())[::-1]
    assert not np.array_equal(c.T["block_table"], cr.T["block_table"][::-1])  # really relabelled
    assert np.abs(got - got_rev).max() < 1e-6
    _cmp("order", got, attention.decode(wl, 0), prefix + tail + 7 * n)


@pytest.mark.parametrize("name", ["small_round", "tiny_q4"])
def test_physical_relabel_bit_exact(name):
    """Moving every physical block to another id (pool rows and the plan's block
    ids permuted together) changes only addresses: the output is bit-identical.
    small_round has shifted segments and deltas; tiny_q4 exercises the Q4 pools
    and their (scale, zero) params."""
    import torch
    wl = spec.make(name)
    c = Case(wl)
    got = c.run(0)
    a = c.T.arrays
    n = int(a["n_phys"])
    sigma = np.random.default_rng(5).permutation(n).astype(np.int32)
    arr = dict(a)
    arr["plan_blocks"] = sigma[a["plan_blocks"]]
    ntok = np.empty_like(a["phys_ntok"])
    ntok[sigma] = a["phys_ntok"]
    arr["phys_ntok"] = ntok

    class Relabelled:
        arrays = arr

    plan2 = K.DevicePlan(Relabelled)
    idx = torch.from_numpy(sigma.astype(np.int64)).cuda()

    def moved(t):
        if t is None:
            return None
        u = torch.empty_like(t)
        u[:, idx] = t
        return u

    k2, v2, kp2, vp2 = moved(c.pool.k), moved(c.pool.v), moved(c.pool.kp), moved(c.pool.vp)
    out2 = torch.empty_like(c.out)
    ws2 = torch.empty_like(c.ws)
    K.paged_decode_attn(wl.shape, plan2, c.q(0), k2, v2, out2, ws2, layer=0, k_params=kp2, v_params=vp2)
    torch.cuda.synchronize()
    got2 = out2.cpu().numpy().astype(np.float64)
    assert not np.array_equal(sigma, np.arange(n))
    assert np.array_equal(got, got2)


def test_deterministic_and_workspace_independent():
    """Two calls give bit-identical outputs, whatever the workspace held before."""
    import torch
    wl = spec.make("small_round")
    c = Case(wl)
    q = c.q(0)
    one = c.run(0, q=q)
    c.ws.fill_(0xFF)  # NaN bit patterns everywhere
    two = c.run(0, q=q)
    assert np.array_equal(one, two)
