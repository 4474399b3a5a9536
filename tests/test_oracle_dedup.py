"""Pins of oracle/dedup.py on hand-built cases whose tables are written out by
hand from the rules (INMS walkthrough sec. 2.2/3.2; TokenDance write-up sec. 1/3).
Each case is chosen so that one plausible mistake fails it: a dropped tier or
group in the key, a missing chain (prefix fork), segment chaining, positional
instead of content indexing, refcount not decremented under a delta, wrong
delta numbering, wrong frame of a delta."""
import numpy as np
import pytest

from oracle import dedup
from workload.spec import GLOBAL, GROUP, PRIVATE, PREFIX, SEGMENT, Agent, Span

B = 4


def toks(*xs):
    return np.array(xs, np.int32)


A = toks(1, 2, 3, 4)
Bt = toks(5, 6, 7, 8)
C = toks(9, 10, 11, 12)
D = toks(13, 14)


def build(agents):
    return dedup.build_tables(B, agents)


def test_shared_prefix_then_private():
    ag = [Agent([Span(GLOBAL, 0, PREFIX, np.concatenate([A, Bt])), Span(PRIVATE, 0, PREFIX, C)]),
          Agent([Span(GLOBAL, 0, PREFIX, np.concatenate([A, Bt])), Span(PRIVATE, 0, PREFIX, C)])]
    T = build(ag)
    assert T["block_table"].tolist() == [[0, 1, 2], [0, 1, 3]]  # identical private tails stay apart
    assert T["refcount"].tolist() == [2, 2, 1, 1]
    assert T["src_pos0"].tolist() == [0, 4, 8, 8]
    assert T["shift"].tolist() == [[0, 0, 0], [0, 0, 0]]
    assert T["phys_agent"].tolist() == [0, 0, 0, 1]
    assert T["phys_block"].tolist() == [0, 1, 2, 2]


def test_tier_and_group_isolate():
    ag = [Agent([Span(GLOBAL, 0, PREFIX, A)]), Agent([Span(GROUP, 1, PREFIX, A)]),
          Agent([Span(GROUP, 2, PREFIX, A)]), Agent([Span(GROUP, 1, PREFIX, A)]),
          Agent([Span(GLOBAL, 5, PREFIX, A)])]  # group id is ignored for GLOBAL
    T = build(ag)
    assert T["block_table"][:, 0].tolist() == [0, 1, 2, 1, 0]
    assert T["refcount"].tolist() == [2, 2, 1]


def test_prefix_fork_breaks_chain():
    # agent 1 differs in block 0, so its block 1 is not shared even though its tokens match
    ag = [Agent([Span(GLOBAL, 0, PREFIX, np.concatenate([A, Bt]))]),
          Agent([Span(GLOBAL, 0, PREFIX, np.concatenate([C, Bt]))])]
    T = build(ag)
    assert T["block_table"].tolist() == [[0, 1], [2, 3]]


def test_segments_are_content_indexed_and_shifted():
    # same segment after private histories of different lengths
    ag = [Agent([Span(PRIVATE, 0, PREFIX, A), Span(GROUP, 0, SEGMENT, np.concatenate([Bt, D]))]),
          Agent([Span(PRIVATE, 0, PREFIX, np.concatenate([A, C, D])), Span(GROUP, 0, SEGMENT, np.concatenate([Bt, D]))])]
    T = build(ag)
    # agent 0: [p0, s0, s1]; agent 1: [p, p, p(partial), s0, s1]
    assert T["block_table"].tolist() == [[0, 1, 2, -1, -1], [3, 4, 5, 1, 2]]
    assert T["ntok"].tolist() == [[4, 4, 2, 0, 0], [4, 4, 2, 4, 2]]
    assert T["dst_pos0"].tolist() == [[0, 4, 8, 0, 0], [0, 4, 8, 10, 14]]
    assert T["src_pos0"].tolist() == [0, 4, 8, 0, 4, 8]
    assert T["shift"][1].tolist() == [0, 0, 0, 6, 6]
    assert T["refcount"].tolist() == [1, 2, 2, 1, 1, 1]


def test_segment_chain_restarts_but_prefix_chain_does_not():
    # the same 4 tokens as a PREFIX block after different histories are different
    # content; as the first block of a SEGMENT they are the same content
    ag = [Agent([Span(GROUP, 0, PREFIX, A), Span(GROUP, 0, PREFIX, Bt)]),
          Agent([Span(GROUP, 0, PREFIX, C), Span(GROUP, 0, PREFIX, Bt)]),
          Agent([Span(GROUP, 0, PREFIX, A), Span(GROUP, 0, SEGMENT, Bt)]),
          Agent([Span(GROUP, 0, PREFIX, C), Span(GROUP, 0, SEGMENT, Bt)])]
    T = build(ag)
    assert T["block_table"].tolist() == [[0, 1], [2, 3], [0, 4], [2, 4]]


def test_repeated_segment_inside_one_agent():
    ag = [Agent([Span(GROUP, 3, SEGMENT, A), Span(PRIVATE, 0, PREFIX, D), Span(GROUP, 3, SEGMENT, A)])]
    T = build(ag)
    assert T["block_table"].tolist() == [[0, 1, 0]]
    assert T["refcount"].tolist() == [2, 1]
    assert T["shift"].tolist() == [[0, 0, 6]]


def test_deltas_ids_refcounts_and_frames():
    seg = np.concatenate([A, Bt, C])
    ag = [Agent([Span(PRIVATE, 0, PREFIX, D), Span(GROUP, 0, SEGMENT, seg)]),
          Agent([Span(PRIVATE, 0, PREFIX, A), Span(GROUP, 0, SEGMENT, seg)], toks(1, 3)),
          Agent([Span(PRIVATE, 0, PREFIX, Bt), Span(GROUP, 0, SEGMENT, seg)], toks(2))]
    T = build(ag)
    # ids: agent0 -> p0=0, seg 1,2,3 ; agent1 private 4 ; agent2 private 5 ; deltas 6,7 (agent1 b1,b3), 8 (agent2 b2)
    assert T["block_table"].tolist() == [[0, 1, 2, 3], [4, 1, 2, 3], [5, 1, 2, 3]]
    assert T["delta_table"].tolist() == [[-1, -1, -1, -1], [-1, 6, -1, 7], [-1, -1, 8, -1]]
    assert T["n_dedup"] == 6 and T["n_delta"] == 3 and T["n_phys"] == 9
    assert T["refcount"].tolist() == [1, 2, 2, 2, 1, 1, 1, 1, 1]
    # deltas are stored in their master's frame
    assert T["src_pos0"].tolist() == [0, 2, 6, 10, 0, 0, 2, 10, 6]
    assert T["shift"].tolist() == [[0, 0, 0, 0], [0, 2, 2, 2], [0, 2, 2, 2]]
    assert T["phys_agent"][6:].tolist() == [1, 1, 2]
    assert T["phys_block"][6:].tolist() == [1, 3, 2]


@pytest.mark.parametrize("deltas,code", [
    (toks(2, 1), dedup.EINVAL),      # unsorted
    (toks(1, 1), dedup.EINVAL),      # repeated
    (toks(4), dedup.EINVAL),         # out of range
    (toks(-1), dedup.EINVAL),
    (toks(0), dedup.EINVAL),         # a private block
])
def test_delta_errors(deltas, code):
    ag = [Agent([Span(PRIVATE, 0, PREFIX, A), Span(GROUP, 0, SEGMENT, np.concatenate([Bt, C, D]))], deltas)]
    with pytest.raises(dedup.OracleError) as e:
        build(ag)
    assert e.value.code == code


def test_delta_on_prefix_block_rejected():
    ag = [Agent([Span(GLOBAL, 0, PREFIX, A)], toks(0))]
    with pytest.raises(dedup.OracleError) as e:
        build(ag)
    assert e.value.code == dedup.EINVAL


def test_group_without_id():
    with pytest.raises(dedup.OracleError) as e:
        build([Agent([Span(GROUP, -1, PREFIX, A)])])
    assert e.value.code == dedup.ETIER


def test_empty_agent_and_empty_span():
    ag = [Agent([]), Agent([Span(GLOBAL, 0, PREFIX, toks()), Span(GLOBAL, 0, PREFIX, A)])]
    T = build(ag)
    assert T["n_blocks"].tolist() == [0, 1]
    assert T["block_table"].tolist() == [[-1], [0]]


def test_brute_force_equivalence_random():
    """Equal ids <=> equal (root kind, then per block domain and tokens, from the
    chain root through the block), checked by brute force over random small
    workloads.  The agent start and a segment start are different roots."""
    rng = np.random.default_rng(5)
    for trial in range(30):
        agents = []
        vocab = [toks(*rng.integers(1, 4, size=rng.integers(1, 9))) for _ in range(4)]
        for j in range(rng.integers(1, 5)):
            spans = []
            for _ in range(rng.integers(1, 4)):
                spans.append(Span(int(rng.integers(0, 3)), int(rng.integers(0, 2)), int(rng.integers(0, 2)),
                                  vocab[rng.integers(0, 4)]))
            agents.append(Agent(spans))
        T = build(agents)
        # brute-force content identity per logical block
        ident = []
        for j, ag in enumerate(agents):
            hist = [("agent-root",)]
            for si, sp in enumerate(ag.spans):
                if sp.kind == SEGMENT:
                    hist = [("segment-root",)]
                dom = (sp.tier, sp.group if sp.tier == GROUP else 0, (j, si) if sp.tier == PRIVATE else None)
                t = list(sp.tokens)
                for t0 in range(0, len(t), B):
                    hist = hist + [(dom, tuple(t[t0:t0 + B]))]
                    ident.append(((j, len([x for x in ident if x[0][0] == j])), tuple(hist)))
        ids = {}
        for (j, b), h in ident:
            ids.setdefault(h, set()).add(T["block_table"][j, b])
        assert all(len(v) == 1 for v in ids.values())
        assert len(ids) == T["n_dedup"]
