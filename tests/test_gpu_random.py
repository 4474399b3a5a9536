"""Seeded random rounds on the GPU against the oracle: head_dim 64 / 128, 16- or
256-token blocks, bf16 or Q4, GQA groups 1..8, 2..12 agents with a global
prefix, private histories and shared segments in per-agent orders, deltas on
segment blocks, partial blocks everywhere; GQA groups up to 16, odd kv-head
counts and kv-head counts of 8 and 16 (XCD-pinned launch mapping) in the extra
cases.  Between them the cases reach every
row class of the planner: one-row and few-row VALU items, narrow and wide
(one and two row tiles per wave) matrix-core items, and the Q4 paths."""
import numpy as np
import pytest

from oracle import attention
from workload import spec

from .gpu_util import Case, log
from .tolerances import ATOL, gate

pytestmark = pytest.mark.gpu

_HEADS = [(4, 4), (8, 4), (8, 2), (16, 4), (10, 2), (32, 4), (16, 2)]


def random_round(seed: int, q4=None, heads=None) -> spec.Workload:
    g = np.random.default_rng(np.random.SeedSequence([seed, 901]))
    d = int(g.choice([64, 128]))
    B = int(g.choice([16, 256]))
    q4_draw = bool(g.random() < 0.35)
    q4 = q4_draw if q4 is None else q4
    h_draw = _HEADS[int(g.integers(len(_HEADS)))]
    hq, hkv = h_draw if heads is None else heads
    n = int(g.integers(2, 13))
    tk = lambda m: g.integers(1, 1 << 30, m).astype(np.int32)
    prefix = tk(int(g.integers(0, 3 * B // 2 + 40)))
    segs = [tk(int(g.integers(1, B + 60))) for _ in range(int(g.integers(0, 4)))]
    agents = []
    for _ in range(n):
        spans = []
        if len(prefix):
            spans.append(spec.Span(spec.GLOBAL, 0, spec.PREFIX, prefix))
        if g.random() < 0.9:
            spans.append(spec.Span(spec.PRIVATE, 0, spec.PREFIX, tk(int(g.integers(1, 2 * B + 30)))))
        for si in g.permutation(len(segs)):
            spans.append(spec.Span(spec.GROUP, 3, spec.SEGMENT, segs[int(si)]))
        agents.append(spec.Agent(spans))
    wl = spec.describe(spec.Workload(f"random{seed}", seed, spec.Shape(1, hq, hkv, d, B,
                                                                       spec.Q4G64 if q4 else spec.BF16, 1e4), agents))
    # deltas on some segment blocks of every agent but the first
    for j in range(1, n):
        ids = spec.segment_block_ids(wl, j)
        if len(ids) and g.random() < 0.7:
            k = int(g.integers(1, len(ids) + 1))
            wl.agents[j].delta_blocks = np.sort(g.choice(ids, size=k, replace=False)).astype(np.int32)
    return spec.describe(wl)


# the seeds, then Q4 at one and two rows per consumer, the largest GQA group (16,
# one kv head) in bf16 and Q4, and an odd kv-head count (windowed unit mapping);
# then kv-head counts that are multiples of 8, which take the launch mapping that
# pins whole kv heads to XCDs: every row class there (VALU, narrow, wide with one
# and two row tiles per wave, both Q4 paths), at 8 and 16 kv heads
_CASES = [(s, None, None) for s in range(16)] + [(100, True, (4, 4)), (101, True, (2, 2)), (102, False, (16, 1)),
                                                  (103, True, (16, 1)), (104, False, (12, 3)), (105, True, (6, 3))]
_CASES += [(106, False, (8, 8)), (107, True, (8, 8)), (108, False, (40, 8)), (109, False, (32, 16)),
           (110, True, (32, 16)), (111, False, (16, 16)), (112, True, (40, 8)), (113, False, (40, 8)),
           (114, False, (64, 8)), (116, False, (64, 8)), (121, False, (128, 16)), (128, False, (128, 16))]
# the two-tile bf16 path at 6 and 7 rows (with masks and shifted consumers), the
# four-tile Q4 path at 3 rows
_CASES += [(200, True, (3, 1)), (200, False, (7, 1)), (205, False, (8, 8)), (211, False, (8, 8))]


def masked_q4_round(seed: int, d: int, B: int) -> spec.Workload:
    """Four Q4 agents that place one shared segment at the same position (after a
    shared prefix), so its blocks are read unshifted by all of them, with deltas
    on some of its blocks for three of them: items of up to 4 one-row consumers
    whose consumer masks skip some blocks (the four-tile Q4 path with masks)."""
    g = np.random.default_rng(np.random.SeedSequence([seed, 907]))
    tk = lambda m: g.integers(1, 1 << 30, m).astype(np.int32)
    prefix = tk(int(g.integers(1, 2 * B)))
    seg = tk(int(g.integers(3 * B, 6 * B)))
    agents = [spec.Agent([spec.Span(spec.GLOBAL, 0, spec.PREFIX, prefix), spec.Span(spec.GROUP, 3, spec.SEGMENT, seg)])
              for _ in range(4)]
    wl = spec.describe(spec.Workload(f"maskedq4_{seed}", seed, spec.Shape(1, 4, 4, d, B, spec.Q4G64, 1e4), agents))
    for j in range(1, 4):
        ids = spec.segment_block_ids(wl, j)
        k = int(g.integers(1, len(ids)))
        wl.agents[j].delta_blocks = np.sort(g.choice(ids, size=k, replace=False)).astype(np.int32)
    return spec.describe(wl)


_MASKED_Q4 = [(0, 128, 16), (1, 64, 16), (2, 128, 256)]


@pytest.mark.parametrize("seed,d,B", _MASKED_Q4)
def test_masked_q4_round(seed, d, B):
    wl = masked_q4_round(seed, d, B)
    L = max(wl.context_len(j) for j in range(wl.n_agents))
    got = Case(wl).run(0)
    ref = attention.decode(wl, 0)
    err = float(np.abs(got - ref).max())
    log(f"masked q4 {seed} d {d} B {B}: max-abs {err:.3e}")
    assert np.isfinite(got).all() and err <= ATOL and err <= gate(ref, L)


@pytest.mark.parametrize("seed,q4,heads", _CASES)
def test_random_round(seed, q4, heads):
    wl = random_round(seed, q4, heads)
    sh = wl.shape
    L = max([wl.context_len(j) for j in range(wl.n_agents)] + [1])
    log(f"seed {seed}: {wl.n_agents} agents, Hq {sh.n_q_heads} / Hkv {sh.n_kv_heads} x {sh.head_dim}, "
        f"B {sh.block_tokens}, {'q4' if sh.kv_dtype == spec.Q4G64 else 'bf16'}, contexts up to {L}")
    c = Case(wl)
    items = c.T.arrays["items"].reshape(-1, 8)
    log(f"  items {len(items)}, rows {sorted(set(items[:, 7].tolist()))}")
    got = c.run(0)
    ref = attention.decode(wl, 0)
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    log(f"  max-abs {err:.3e}")
    assert np.isfinite(got).all()
    for j in range(wl.n_agents):
        if wl.context_len(j) == 0:
            assert not got[j].any()
    assert err <= ATOL and err <= gate(ref, L)
