"""Pins of oracle/attention.py: brute force, a library special case, closed
forms (constant V, needle), the sharing invariance (TokenDance write-up,
evaluation: sharing adds no error), and the power of the parity gate (planted
mistakes must exceed the tolerance the GPU tests use)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, dedup, rope
from workload import rng, spec

from .tolerances import ATOL, gate


def brute(q, K, V, scale):
    Hq, d = q.shape
    L, Hkv, _ = K.shape
    grp = Hq // Hkv
    out = np.zeros((Hq, d))
    for h in range(Hq):
        g = h // grp
        s = [sum(float(K[t, g, i]) * float(q[h, i]) for i in range(d)) * scale for t in range(L)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = sum(w)
        for i in range(d):
            out[h, i] = sum(w[t] * float(V[t, g, i]) for t in range(L)) / tot
    return out


def test_brute_force_small():
    r = np.random.default_rng(0)
    q = r.standard_normal((4, 8))
    K = r.standard_normal((11, 2, 8))
    V = r.standard_normal((11, 2, 8))
    assert np.abs(attention.attend(q, K, V, 0.3) - brute(q, K, V, 0.3)).max() < 1e-12


def test_matches_torch_sdpa_single_agent():
    """One agent, no sharing, no shift: torch's scaled_dot_product_attention
    (float64, CPU) on the dense tensors, GQA expanded by repeat_interleave."""
    wl = spec.make("tiny")
    j = 2
    store = attention._Store(wl, 0)
    K, V = attention.dense_plain(wl, j, store, [0, 1])
    q = rng.bf16_bits_to_f32(spec.q_bits(wl, 0)[j]).astype(np.float64)
    out = attention.attend(q, K, V, 1 / math.sqrt(64))
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(2, dim=0)  # [Hq, L, d]
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(2, dim=0)
    qt = torch.from_numpy(q)[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)[:, 0, :].numpy()
    assert np.abs(out - ref).max() < 1e-12


def test_constant_v():
    r = np.random.default_rng(1)
    q = r.standard_normal((2, 16))
    K = r.standard_normal((50, 1, 16))
    V = np.tile(r.standard_normal(16), (50, 1, 1))
    assert np.abs(attention.attend(q, K, V, 0.25) - V[0, 0]).max() < 1e-14


def test_needle():
    """k_n = 40 sqrt(d) q/|q|^2 gives a scaled score of 40 against N(0,1) others."""
    r = np.random.default_rng(2)
    d, L = 64, 4000
    q = r.standard_normal((1, d))
    K = r.standard_normal((L, 1, d))
    V = r.standard_normal((L, 1, d))
    K[1234, 0] = 40 * math.sqrt(d) * q[0] / (q[0] @ q[0])
    out = attention.attend(q, K, V, 1 / math.sqrt(d))
    assert np.abs(out[0] - V[1234, 0]).max() < L * math.exp(-30)


def test_empty_context_is_zero():
    q = np.ones((2, 4))
    assert not attention.attend(q, np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), 1.0).any()


@pytest.mark.parametrize("name", ["tiny", "tiny_seg", "tiny_q4", "small_round"])
def test_sharing_invariance(name):
    """Materialising through the dedup tables (each physical block stored once,
    deltas overlaid, keys moved by the table's shift) gives bit-identical dense
    attention to materialising each agent's logical context directly."""
    wl = spec.make(name)
    T = dedup.build_tables(wl.shape.block_tokens, wl.agents)
    a = attention.decode(wl)
    b = attention.decode(wl, tables=T)
    assert np.array_equal(a, b)


def _planted(wl, mistake):
    """Oracle output with one planted mistake (CPU only), for gate power."""
    T = dedup.build_tables(wl.shape.block_tokens, wl.agents)
    T2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in T.items()}
    if mistake == "drop_block":
        j = 1
        b = int(T2["n_blocks"][j]) // 2
        T2["n_blocks"] = T2["n_blocks"].copy()
        bt = list(range(int(T2["n_blocks"][j])))
        bt.pop(b)
        for key in ("block_table", "delta_table", "shift"):
            row = T2[key][j].copy()
            T2[key][j, : len(bt)] = row[bt]
        T2["n_blocks"][j] -= 1
    elif mistake == "ignore_delta":
        T2["delta_table"][:] = -1
    elif mistake == "flip_shift":
        T2["shift"] = -T2["shift"]
    return attention.decode(wl, tables=T2)


@pytest.mark.parametrize("name,mistake", [("tiny_seg", "drop_block"), ("tiny_seg", "ignore_delta"),
                                          ("tiny_seg", "flip_shift"), ("tiny", "drop_block"),
                                          ("small_round", "flip_shift"), ("small_round", "ignore_delta")])
def test_gate_has_power(name, mistake):
    wl = spec.make(name)
    good = attention.decode(wl)
    bad = _planted(wl, mistake)
    err = np.abs(good - bad).max()
    L = max(wl.context_len(j) for j in range(wl.n_agents))
    assert err > ATOL and err > gate(good, L)


def test_gqa_head_mapping_matters():
    wl = spec.make("tiny")
    store = attention._Store(wl, 0)
    K, V = attention.dense_plain(wl, 0, store, [0, 1])
    q = rng.bf16_bits_to_f32(spec.q_bits(wl, 0)[0]).astype(np.float64)
    good = attention.attend(q, K, V, 0.125)
    bad = attention.attend(q, K[:, ::-1], V[:, ::-1], 0.125)  # wrong kv head per q head
    assert np.abs(good - bad).max() > ATOL
