"""The C-ABI library on the CPU (no GPU calls): it loads and exports every
symbol include/kvpool.h declares, and kvpool_build_tables is bit-exact with the
oracle on tables, refcounts, delta ids and shifts for every config, under
forced hash collisions, and on the error cases."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import dedup
from shared_paged_kv_amd import _lib as K
from workload import spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE_KEYS = ["n_blocks", "block_table", "delta_table", "ntok", "dst_pos0", "shift", "src_pos0", "refcount",
              "phys_ntok", "phys_agent", "phys_block"]


def test_exports_every_declared_symbol():
    inc = os.path.join(ROOT, "include")
    declared = set()
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            hdr = open(os.path.join(inc, f)).read()
            declared |= set(re.findall(r"^\w[\w\s\*]*?\b(\w+)\s*\(", hdr, re.M)) - {"if", "return"}
    assert declared == set(K.EXPORTS)
    L = C.CDLL(K.LIB_PATH)
    for s in declared:
        assert hasattr(L, s), s


def test_checked_build_exports_and_reports():
    """The checked build (kernels with bounds checks on table indices) exports
    the same symbols and says that it is the checked one; the ordinary build
    says it is not."""
    L = C.CDLL(os.path.join(ROOT, "shared_paged_kv_amd", "libkvpool_checked.so"))
    for s in K.EXPORTS:
        assert hasattr(L, s), s
    assert L.kvpool_device_checks_enabled() == 1
    assert C.CDLL(os.path.join(ROOT, "shared_paged_kv_amd", "libkvpool.so")).kvpool_device_checks_enabled() == 0


def _same(T, O):
    for k in TABLE_KEYS:
        assert np.array_equal(T[k], O[k]), k
    for k in ("n_phys", "n_dedup", "n_delta"):
        assert T.arrays[k] == O[k]


@pytest.mark.parametrize("name", ["tiny", "tiny_seg", "tiny_q4", "small_round", "inms", "tokendance", "q4"])
def test_tables_bit_exact(name):
    wl = spec.make(name)
    _same(K.build_tables(wl.shape, wl.agents), dedup.build_tables(wl.shape.block_tokens, wl.agents))


@pytest.mark.slow
def test_tables_bit_exact_scale():
    wl = spec.make("scale")
    _same(K.build_tables(wl.shape, wl.agents), dedup.build_tables(wl.shape.block_tokens, wl.agents))


def test_forced_hash_collisions_do_not_change_tables():
    wl = spec.make("small_round")
    ref = K.build_tables(wl.shape, wl.agents)
    try:
        K.set_hash_bits(3)
        T = K.build_tables(wl.shape, wl.agents)
    finally:
        K.set_hash_bits(64)
    for k in TABLE_KEYS:
        assert np.array_equal(T[k], ref[k])


def test_fnv1a_words():
    """Offset basis and prime as printed on the shared-memory cache page; one
    32-bit token id per step (h ^= w; h *= prime mod 2^64)."""
    basis, prime = 1469598103934665603, 1099511628211
    assert K.fnv1a64_words([]) == basis
    w = [7, 0xFFFFFFFF, 123456789]
    h = basis
    for x in w:
        h = ((h ^ x) * prime) % 2**64
    assert K.fnv1a64_words(w) == h


def test_brute_force_random_against_oracle():
    """Random small workloads with every tier, kind, repeated tokens, partial
    blocks and deltas: library == oracle bit for bit (or the same error code)."""
    r = np.random.default_rng(11)
    for trial in range(60):
        vocab = [r.integers(1, 4, size=r.integers(0, 40)).astype(np.int32) for _ in range(5)]
        agents = []
        for j in range(r.integers(1, 6)):
            spans = [spec.Span(int(r.integers(0, 3)), int(r.integers(0, 3)), int(r.integers(0, 2)), vocab[r.integers(0, 5)])
                     for _ in range(r.integers(0, 4))]
            agents.append(spec.Agent(spans))
        shape = spec.Shape(1, 4, 2, 64, 16)
        # deltas on some shared segment blocks
        try:
            O = dedup.build_tables(16, agents)
        except dedup.OracleError:
            continue
        for j, ag in enumerate(agents):
            cand = []
            b = 0
            for sp in ag.spans:
                nb = -(-len(sp.tokens) // 16)
                if sp.kind == spec.SEGMENT and sp.tier != spec.PRIVATE:
                    cand += list(range(b, b + nb))
                b += nb
            if cand and r.random() < 0.5:
                ag.delta_blocks = np.array(sorted(r.choice(cand, size=min(len(cand), 2), replace=False)), np.int32)
        O = dedup.build_tables(16, agents)
        _same(K.build_tables(shape, agents), O)


@pytest.mark.parametrize("mut,code", [
    (lambda a: setattr(a[0], "delta_blocks", np.array([5, 4], np.int32)), dedup.EINVAL),
    (lambda a: setattr(a[0], "delta_blocks", np.array([0], np.int32)), dedup.EINVAL),
    (lambda a: setattr(a[0], "delta_blocks", np.array([999], np.int32)), dedup.EINVAL),
    (lambda a: setattr(a[0].spans[1], "group", -3), dedup.ETIER),
    (lambda a: setattr(a[0].spans[1], "kind", 7), dedup.EINVAL),
])
def test_error_codes_match_oracle(mut, code):
    wl = spec.make("tiny_seg")
    agents = wl.agents
    mut(agents)
    with pytest.raises(dedup.OracleError) as e:
        dedup.build_tables(16, agents)
    assert e.value.code == code
    with pytest.raises(K.KvpError) as e2:
        K.build_tables(wl.shape, agents)
    assert e2.value.code == code


@pytest.mark.parametrize("field,val", [("head_dim", 96), ("block_tokens", 32), ("n_q_heads", 3),
                                       ("kv_dtype", 5), ("rope_theta", 0.0), ("n_layers", 0)])
def test_bad_shape(field, val):
    wl = spec.make("tiny")
    setattr(wl.shape, field, val)
    with pytest.raises(K.KvpError) as e:
        K.build_tables(wl.shape, wl.agents)
    assert e.value.code == K.KVP_EINVAL


def test_decode_argument_errors_without_launch():
    """Argument checks happen before anything is enqueued (no GPU needed)."""
    wl = spec.make("tiny")
    T = K.build_tables(wl.shape, wl.agents)
    a = T.arrays
    pl = K.kvp_plan_dev()
    pl.n_agents, pl.n_phys, pl.n_items = a["n_agents"], a["n_phys"], a["items"].shape[0]
    pl.n_qcons, pl.n_part_rows, pl.n_qcons_shifted = a["n_qcons"], a["n_part_rows"], a["n_qcons_shifted"]
    for i in range(6):
        pl.class_items[i] = int(a["class_items"][i])
    pl.unit_span = int(a["unit_span"])
    for f in K.PLAN_ARRAYS:
        setattr(pl, f, 16)
    sh = K.make_shape(wl.shape)
    L = K.lib()
    n = C.c_size_t()
    assert L.paged_decode_attn_workspace_bytes(C.byref(sh), C.byref(pl), C.byref(n)) == 0
    need = n.value
    x = C.c_void_p(4096)
    assert L.paged_decode_attn(C.byref(sh), C.byref(pl), x, x, x, None, None, 0, 0.125, x, x, need - 1, None) == K.KVP_EWORKSPACE
    assert L.paged_decode_attn(C.byref(sh), C.byref(pl), x, x, x, None, None, 1, 0.125, x, x, need, None) == K.KVP_EINVAL
    assert L.paged_decode_attn(C.byref(sh), C.byref(pl), None, x, x, None, None, 0, 0.125, x, x, need, None) == K.KVP_EINVAL
    # a pool, out or workspace the call would use may not be NULL
    assert L.paged_decode_attn(C.byref(sh), C.byref(pl), x, None, x, None, None, 0, 0.125, x, x, need, None) == K.KVP_EINVAL
    assert L.paged_decode_attn(C.byref(sh), C.byref(pl), x, x, x, None, None, 0, 0.125, None, x, need, None) == K.KVP_EINVAL
    assert L.paged_decode_attn(C.byref(sh), C.byref(pl), x, x, x, None, None, 0, 0.125, x, None, need, None) == K.KVP_EINVAL
    pl.class_items[0] += 1
    assert L.paged_decode_attn(C.byref(sh), C.byref(pl), x, x, x, None, None, 0, 0.125, x, x, need, None) == K.KVP_EINVAL
    pl.class_items[0] -= 1
    # a plan without agents uses no pointer: nothing is enqueued, KVP_OK
    pl.n_agents = pl.n_items = pl.n_qcons = pl.n_part_rows = pl.n_qcons_shifted = 0
    for i in range(6):
        pl.class_items[i] = 0
    assert L.paged_decode_attn(C.byref(sh), C.byref(pl), None, None, None, None, None, 0, 0.125, None, None, 0,
                               None) == K.KVP_OK
    assert L.paged_decode_attn(C.byref(sh), C.byref(pl), None, None, None, None, None, 1, 0.125, None, None, 0,
                               None) == K.KVP_EINVAL  # arguments are still checked
    assert L.kv_rerotate(x, x, x, 4, 2, 63, 1e4, 0, 0, None) == K.KVP_EINVAL
    assert L.kv_rerotate(x, x, x, 4, 2, 64, 1e4, 0, 2, None) == K.KVP_EINVAL  # in place, different dtypes



def test_binding_refuses_bad_tensors_before_the_call():
    """The binding checks what the library cannot see -- device placement,
    contiguity, dtype and extent of every tensor -- and raises before any
    pointer is passed (CPU tensors stand in for device ones here)."""
    import torch
    wl = spec.make("tiny")
    T = K.build_tables(wl.shape, wl.agents)
    a = T.arrays

    class Plan:  # DevicePlan's counts without the device copies
        c = K.kvp_plan_dev()

    Plan.c.n_agents, Plan.c.n_phys, Plan.c.n_items = a["n_agents"], a["n_phys"], a["items"].shape[0]
    sh = wl.shape
    rows = (a["n_agents"], sh.n_q_heads, sh.head_dim)
    pool = (sh.n_layers, a["n_phys"], sh.n_kv_heads, sh.block_tokens, sh.head_dim)
    q = torch.zeros(rows, dtype=torch.bfloat16)
    out = torch.zeros(rows, dtype=torch.float32)
    kp = torch.zeros(pool, dtype=torch.bfloat16)
    ws = torch.zeros(16, dtype=torch.uint8)

    def refused(match, **kw):
        args = dict(q=q, k_pool=kp, v_pool=kp, out=out, workspace=ws)
        args.update(kw)
        with pytest.raises(K.KvpError, match=match):
            K.paged_decode_attn(sh, Plan, args["q"], args["k_pool"], args["v_pool"], args["out"], args["workspace"])

    refused("q: dtype", q=q.float())
    refused("k_pool: dtype", k_pool=kp.half())
    refused("out: dtype", out=out.to(torch.bfloat16))
    refused("q: .* elements", q=q[:-1])
    refused("k_pool: .* elements", k_pool=kp[:, :-1])
    refused("v_pool: dtype", v_pool=kp.to(torch.uint8))
    refused("v_pool: required", v_pool=None)
    refused("device memory")  # every tensor is a host tensor here
    with pytest.raises(K.KvpError, match="contiguous"):
        K._ptr(torch.zeros(4, 4).t())
    x = torch.zeros(3, 2, 64, dtype=torch.bfloat16)
    s32 = torch.zeros(3, dtype=torch.int32)
    for bad, match in ((dict(shift=s32[:2]), "shift: .* elements"), (dict(shift=s32.long()), "shift: dtype"),
                       (dict(x=x.half()), "x: dtype"), (dict(x=x[0]), r"x: expected \[rows"),
                       (dict(), "device memory")):
        args = dict(x=x, shift=s32)
        args.update(bad)
        with pytest.raises(K.KvpError, match=match):
            K.kv_rerotate(args["x"], args["shift"], 1e4)

def check_plan_coverage(a, grp):
    """Every (agent, logical block) of tables a is read by exactly one (item,
    consumer) with its shift; overlaid masters only through masked slots."""
    seen = {}
    for it in a["items"]:
        b0, b1, c0, c1, pbase, mbase, mstride, rows = [int(x) for x in it]
        assert rows == (c1 - c0) * grp
        for bi in range(b0, b1):
            p = int(a["plan_blocks"][bi])
            for c in range(c0, c1):
                if mbase >= 0:
                    w = a["mask"][mbase + (bi - b0) * mstride + (c - c0) // 32]
                    if not (w >> ((c - c0) % 32)) & 1:
                        continue
                qc = int(a["cons"][c])
                j, s = int(a["qcons"][2 * qc]), int(a["qcons"][2 * qc + 1])
                seen[(j, p, s)] = seen.get((j, p, s), 0) + 1
    want = {}
    for j in range(a["n_agents"]):
        for b in range(int(a["n_blocks"][j])):
            e = a["delta_table"][j, b] if a["delta_table"][j, b] >= 0 else a["block_table"][j, b]
            key = (j, int(e), int(a["shift"][j, b]))
            want[key] = want.get(key, 0) + 1
    assert seen == want


def test_plan_covers_every_effective_reference():
    """Host-side check of the work plan: every (agent, logical block) is read by
    exactly one (item, consumer) with the right shift, and masked otherwise; the
    partial rows and combine lists are consistent (check_plan_partials)."""
    for name in ["tiny_seg", "small_round", "tokendance", "q4"]:
        wl = spec.make(name)
        T = K.build_tables(wl.shape, wl.agents)
        check_plan_coverage(T.arrays, wl.shape.n_q_heads // wl.shape.n_kv_heads)
        check_plan_partials(T.arrays, wl.shape.n_q_heads // wl.shape.n_kv_heads)


@pytest.mark.parametrize("name", ["tiny_seg", "small_round", "tiny_q4", "q4"])
def test_plan_lookups_are_derived(name):
    """plan_ntok and cons_row are lookups the device takes in place of a chain of
    two loads: each entry equals what it is derived from (a block's valid tokens;
    a consumer's agent in q, or its index among the shifted consumers' rotated
    copies)."""
    wl = spec.make(name)
    a = K.build_tables(wl.shape, wl.agents).arrays
    assert np.array_equal(a["plan_ntok"], a["phys_ntok"][a["plan_blocks"]])
    nu = a["n_qcons"] - a["n_qcons_shifted"]
    qc = a["cons"]
    want = np.where(qc < nu, a["qcons"].reshape(-1, 2)[qc, 0], qc - nu)
    assert np.array_equal(a["cons_row"], want)
    if name == "small_round":
        assert (qc >= nu).any() and (qc < nu).any()   # both kinds occur


@pytest.mark.parametrize("name", ["tiny_seg", "small_round", "tokendance"])
def test_plan_rotation_table(name):
    """rope_cs holds, for each shifted (agent, shift) pair in qcons order, the cos
    and sin of -shift * theta_i (theta_i = rope_theta^(-2i/d)) rounded to float32
    from float64 -- the rotation R(-shift) the tile pass applies to that
    consumer's query (INMS walkthrough sec. 3.2).  Checked against numpy's float64
    cos and sin, to within one float32 ulp."""
    wl = spec.make(name)
    a = K.build_tables(wl.shape, wl.agents).arrays
    d, ns = wl.shape.head_dim, int(a["n_qcons_shifted"])
    assert ns > 0
    nu = int(a["n_qcons"]) - ns
    shift = a["qcons"].reshape(-1, 2)[nu:, 1].astype(np.float64)
    assert (shift != 0).all()
    theta = float(np.float32(wl.shape.rope_theta)) ** (-2.0 * np.arange(d // 2) / d)
    ang = -shift[:, None] * theta[None, :]
    got = a["rope_cs"].reshape(ns, d // 2, 2)
    for k, want in ((0, np.cos(ang)), (1, np.sin(ang))):
        w32 = want.astype(np.float32)
        ulp = np.spacing(np.abs(w32)).astype(np.float64)
        assert (np.abs(got[..., k].astype(np.float64) - w32) <= ulp).all()


def test_random_rounds_reach_every_kernel_path():
    """The GPU random rounds keep reaching each kernel path and its edge cases
    (the planner decides which path an item takes; this fails if a change to it
    leaves a path or a case untested on the device)."""
    from tests.test_gpu_random import _CASES, _MASKED_Q4, masked_q4_round, random_round
    seen = set()
    rounds = [random_round(*c) for c in _CASES] + [masked_q4_round(*c) for c in _MASKED_Q4]
    for wl in rounds:
        a = K.build_tables(wl.shape, wl.agents).arrays
        nu = a["n_qcons"] - a["n_qcons_shifted"]
        q4 = wl.shape.kv_dtype == spec.Q4G64
        for it in a["items"]:
            rows = int(it[7])
            shifted = bool((a["cons"][it[2]:it[3]] >= nu).any())
            masked = bool(it[5] >= 0)
            if q4:
                path = "q4 valu" if rows == 1 else ("q4 four-tile" if rows <= 4 and not shifted else "q4 one-tile")
            else:
                path = ("valu" if rows <= 4 else "two-tile" if rows <= 7 else "one-tile" if rows <= 16 else
                        "wide 1" if rows <= 64 else "wide 2")
            seen.add((path, "rows", rows if path in ("q4 four-tile", "two-tile") else 0))
            seen.add((path, "masked", masked))
            seen.add((path, "shifted", shifted))
    for want in [("q4 four-tile", "rows", r) for r in (2, 3, 4)] + [("two-tile", "rows", r) for r in (5, 6, 7)]:
        assert want in seen, want
    for path in ("q4 four-tile", "two-tile", "q4 one-tile", "one-tile", "wide 1", "wide 2", "valu", "q4 valu"):
        assert (path, "masked", False) in seen, path
    for path in ("q4 four-tile", "two-tile", "one-tile", "wide 1", "wide 2"):
        assert (path, "masked", True) in seen, path
    for path in ("two-tile", "q4 one-tile", "one-tile", "wide 1", "wide 2"):
        assert (path, "shifted", True) in seen, path


def check_plan_partials(a, grp):
    """The partial rows of the plan: item it writes rows part_base + (c - c0) * grp
    + [0, grp) (per kv head) for its consumer entries c; those ranges tile
    [0, n_part_rows) without overlap, and agent j's combine list holds exactly
    the first row of each of its consumer entries, once, in ascending order."""
    P = int(a["n_part_rows"])
    owner = np.full(P, -1, np.int64)
    want = {j: [] for j in range(int(a["n_agents"]))}
    for k, it in enumerate(a["items"]):
        b0, b1, c0, c1, pbase, mbase, mstride, rows = [int(x) for x in it]
        assert 0 <= pbase and pbase + rows <= P
        assert (owner[pbase:pbase + rows] == -1).all(), "items' partial rows overlap"
        owner[pbase:pbase + rows] = k
        for c in range(c0, c1):
            j = int(a["qcons"][2 * int(a["cons"][c])])
            want[j].append(pbase + (c - c0) * grp)
    assert (owner >= 0).all(), "a partial row no item writes"
    ptr, comb = a["comb_ptr"], a["comb_rows"]
    assert int(ptr[0]) == 0 and int(ptr[-1]) == len(comb)
    for j, rows in want.items():
        got = [int(x) for x in comb[int(ptr[j]):int(ptr[j + 1])]]
        assert got == sorted(rows), j


def test_plan_invariants_on_random_rounds():
    """Every seeded random round of the GPU tests, and a wider sweep of the same
    generator: the plan reads every (agent, logical block) exactly once with its
    shift, its items' partial rows tile the workspace without overlap, and each
    agent's combine list is exactly its consumers' rows (host logic only)."""
    from tests.test_gpu_random import _CASES, _MASKED_Q4, masked_q4_round, random_round
    rounds = [random_round(*c) for c in _CASES] + [masked_q4_round(*c) for c in _MASKED_Q4]
    rounds += [random_round(s) for s in range(1000, 1040)]
    for wl in rounds:
        a = K.build_tables(wl.shape, wl.agents).arrays
        grp = wl.shape.n_q_heads // wl.shape.n_kv_heads
        check_plan_coverage(a, grp)
        check_plan_partials(a, grp)
