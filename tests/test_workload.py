"""The seeded input generator: Philox4x32-10 against the known-answer vectors
published with the Random123 library (Salmon et al., SC'11), bf16 rounding,
value statistics, and the configs' structural recipe."""
import numpy as np

from workload import rng, spec

KAT = [  # (counter, key) -> output, Random123 kat_vectors for philox4x32_10
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


def test_philox_kat():
    for c, k, want in KAT:
        got = rng.philox4x32_10(*[np.uint32(x) for x in c], *[np.uint32(x) for x in k])
        assert tuple(int(x) for x in got) == want


def test_bf16_rne():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-8 + 2**-20], np.float32)
    b = rng.f32_to_bf16_bits(x)
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]
    assert np.array_equal(rng.bf16_bits_to_f32(b)[[0, 3]], x[[0, 3]])


def test_values_exact_and_near_standard_normal():
    w = rng.tile_words((1, 2, 3, 4), 0, 0, 1 << 18)
    v = rng.ih_value(w)
    s = np.round(v * 1024 / 7).astype(np.int64)
    assert np.array_equal(s * 7 / 1024, v.astype(np.float64))  # exact
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0104) < 0.01


def test_streams_disjoint_and_deterministic():
    a = rng.bf16_tile((5, 6, 7, 8), 3, rng.SEL_K, (4, 16))
    assert np.array_equal(a, rng.bf16_tile((5, 6, 7, 8), 3, rng.SEL_K, (4, 16)))
    assert not np.array_equal(a, rng.bf16_tile((5, 6, 7, 8), 3, rng.SEL_V, (4, 16)))
    assert not np.array_equal(a, rng.bf16_tile((5, 6, 7, 8), 4, rng.SEL_K, (4, 16)))
    # a head slice equals the corresponding slice of the full tile
    full = rng.bf16_tile((5, 6, 7, 8), 1, 0, (3, 16, 64))
    assert np.array_equal(rng.bf16_range((5, 6, 7, 8), 1, 0, 2 * 16 * 64, 16 * 64), full[2].reshape(-1))


def test_config_recipes():
    wl = spec.make("inms")
    assert all(wl.context_len(j) == 16384 for j in range(8))
    wl = spec.make("tokendance")
    assert wl.n_agents == 64 and len(wl.agents[0].spans) == 65
    P = [len(a.spans[0].tokens) for a in wl.agents]
    S = [len(s.tokens) for s in wl.agents[0].spans[1:]]
    assert 512 <= min(P) and max(P) <= 4096 and 128 <= min(S) and max(S) <= 512
    assert len(wl.agents[0].delta_blocks) == 0
    for j in range(1, 64):
        nseg = len(spec.segment_block_ids(wl, j))
        f = len(wl.agents[j].delta_blocks) / nseg
        assert 0.025 <= f <= 0.095
        # clustered: every segment's first block is taken before any interior block
    wl = spec.make("q4")
    assert wl.shape.block_tokens == 256 and all(wl.context_len(j) == 8192 for j in range(12))


def test_delta_runs_start_at_segment_boundaries():
    wl = spec.make("small_round")
    B = wl.shape.block_tokens
    for j in range(1, wl.n_agents):
        starts = set()
        b = -(-len(wl.agents[j].spans[0].tokens) // B)
        for s in wl.agents[j].spans[1:]:
            starts.add(b)
            b += -(-len(s.tokens) // B)
        d = set(int(x) for x in wl.agents[j].delta_blocks)
        # either every segment's leading block carries a delta, or all deltas sit in leading runs
        assert starts <= d or all(any(x - k in starts and all(x - i in d for i in range(k + 1))
                                      for k in range(3)) for x in d)
