"""Pins of oracle/footprint.py and the oracle's physical block counts against the
pages' printed worked examples and closed forms."""
import json
import math
import os

import numpy as np
import pytest

from oracle import dedup, footprint, q4
from workload import spec

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "footprint_examples.json")))


def test_inms_per_token_bytes():
    g = G["inms_per_token"]
    assert footprint.kv_bytes_per_token_mha(g["hidden"], g["dtype_bytes"]) == g["per_layer_bytes"]
    assert footprint.kv_bytes_per_token_mha(g["hidden"], g["dtype_bytes"], g["layers"]) == g["per_token_bytes"]


def test_memdecay_per_token_bytes():
    g = G["memdecay_per_token"]
    assert footprint.kv_bytes_per_token_mha(g["hidden"], g["dtype_bytes"]) == g["per_layer_bytes"]


def test_shm_gqa_per_token_and_table():
    g = G["shm_gqa_per_token"]
    per = footprint.kv_bytes_per_token_gqa(g["layers"], g["kv_heads"], g["head_dim"], g["dtype_bytes"])
    assert per == g["per_token_bytes"]
    t = G["shm_table_4096"]
    # the page's table computes tokens * (bytes/1024) / 1000
    assert t["tokens"] * per / 1024 / 1000 == pytest.approx(t["per_request_mb"])
    assert 8 * t["tokens"] * per / 1024 / 1000 == pytest.approx(t["eight_way_mb"])


def test_inms_eight_agent_example():
    g = G["inms_eight_agents"]
    assert footprint.independent(g["n"], g["L"], g["s"]) == g["independent_bytes"]
    assert footprint.shared(g["n"], g["L"], g["s"], g["p"]) == pytest.approx(g["shared_bytes_formula"], rel=1e-12)
    assert footprint.shared(g["n"], g["L"], g["s"], g["p"]) / 2**30 == pytest.approx(30.4, rel=1e-9)


def test_inms_three_agent_example():
    g = G["inms_three_agents"]
    assert footprint.independent(g["n"], g["L"], g["s"]) == pytest.approx(g["independent_bytes"])
    assert footprint.shared(g["n"], g["L"], g["s"], g["p"]) == pytest.approx(g["shared_bytes"], rel=1e-12)


def test_q4_ratio():
    g = G["q4_ratio"]
    r = q4.compression_ratio(g["head_dim"])
    assert r == g["layout_ratio"]
    assert round(r, 3) == g["printed"]


def test_inms_config_block_count_is_closed_form():
    """8 agents x 1024 blocks sharing a 614-block prefix: the INMS closed form with
    p = 614/1024 and L in blocks must give the oracle's physical block count."""
    wl = spec.make("inms")
    T = dedup.build_tables(16, wl.agents)
    assert T["n_phys"] == footprint.shared_prefix_blocks(8, 614, 1024) == 3894
    # and in bytes: unique bytes == closed form with s = bytes per block
    s = 16 * 32 * 128 * 2 * 2
    assert dedup.unique_kv_bytes(T, 32, 128, 0) == 1020788736
    assert dedup.unique_kv_bytes(T, 32, 128, 0) == round(footprint.shared(8, 1024, s, 614 / 1024))


def test_tiny_block_count():
    wl = spec.make("tiny")
    T = dedup.build_tables(16, wl.agents)
    tails = [len(a.spans[1].tokens) for a in wl.agents]
    assert T["n_phys"] == 8 + sum(math.ceil(t / 16) for t in tails)


@pytest.mark.parametrize("name", ["tokendance", "small_round"])
def test_round_block_count_master_plus_mirrors(name):
    """One dense master plus sparse mirrors: private blocks of every agent, every
    segment once, plus one block per delta."""
    wl = spec.make(name)
    B = wl.shape.block_tokens
    T = dedup.build_tables(B, wl.agents)
    priv = sum(math.ceil(len(a.spans[0].tokens) / B) for a in wl.agents)
    segs = sum(math.ceil(len(s.tokens) / B) for s in wl.agents[0].spans[1:])
    deltas = sum(len(a.delta_blocks) for a in wl.agents)
    assert T["n_phys"] == priv + segs + deltas
    assert T["n_delta"] == deltas
    assert int(T["refcount"].sum()) == int(T["n_blocks"].sum())
    # every segment block is referenced by all agents minus those holding a delta on it
    n = wl.n_agents
    for p in range(T["n_dedup"]):
        j0, b0 = T["phys_agent"][p], T["phys_block"][p]
        if wl.agents[j0].spans[wl.blk_span[j0][b0]].tier == spec.GROUP:
            overlaid = int(((T["block_table"] == p) & (T["delta_table"] >= 0)).sum())
            assert T["refcount"][p] == n - overlaid


def test_q4_config_bytes():
    wl = spec.make("q4")
    T = dedup.build_tables(256, wl.agents)
    assert T["n_phys"] == 384
    assert dedup.unique_kv_bytes(T, 8, 128, 1) == 113246208
    assert dedup.unique_kv_bytes(T, 8, 128, 1) == 0.28125 * 402653184
