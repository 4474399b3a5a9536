"""Decode-attention benchmark on one MI355X.

Workload (the metric's headline configuration): 8 agents x 16384-token contexts
sharing a 9824-token global prefix (INMS walkthrough sec. 1.2 shape), one layer of
a 7B-like MHA (32 heads x 128), block 16, bf16 K/V, one decode query per agent.
A step is one paged_decode_attn call per layer (tile pass, then combine)
over the deduplicated pool, inputs resident in HBM.  Each timed step follows an
untimed write and read of 1 GiB that evicts L2 and the MALL, so its KV comes
from HBM.

Prints one JSON line: agent-tokens/s (value: agents over the median timed step),
effective unique-KV GB/s against the 8 TB/s HBM peak, the roofline of the tile
pass (its average launch against 8 TB/s and against a plain read of the same
byte count on this GPU), warm back-to-back steps for information, and the CPU
oracle timed on the host's cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def flush_buffers():
    import torch
    return (torch.empty(1 << 30, dtype=torch.uint8, device="cuda"),
            torch.empty(4096, dtype=torch.int64, device="cuda"))


def flush(scratch, rsum):
    """Evicts L2 and the 256 MB MALL before a timed step: writes 1 GiB of scratch,
    then reads it back.  The read leaves the MALL holding clean lines, so the
    step is not charged for writing back the write's own dirty lines when its
    reads evict them (in a decode loop the MALL holds clean lines of the previous
    layer's reads)."""
    import torch
    scratch.fill_(1)
    torch.sum(scratch.view(torch.int64).view(4096, -1), dim=1, out=rsum)


def gpu_run(cfg, steps, warmup, copy_probe=False):
    import torch

    from shared_paged_kv_amd import _lib as K
    from workload import device as wdev
    from workload import spec

    wl = spec.make(cfg)
    t0 = time.perf_counter()
    T = K.build_tables(wl.shape, wl.agents)
    t_tables = time.perf_counter() - t0
    a = T.arrays
    plan = K.DevicePlan(T)
    pool = wdev.Pool(wl, a["phys_agent"], a["phys_block"], a["phys_ntok"], a["n_dedup"])
    qs = [wdev.fill_q(wl, layer) for layer in range(wl.shape.n_layers)]
    ws = torch.empty(max(1, K.workspace_bytes(wl.shape, plan)), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.n_agents, wl.shape.n_q_heads, wl.shape.head_dim), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    # one step = paged_decode_attn for every layer (one call each)
    def step():
        for layer in range(wl.shape.n_layers):
            K.paged_decode_attn(wl.shape, plan, qs[layer], pool.k, pool.v, out, ws, layer=layer,
                                k_params=pool.kp, v_params=pool.vp)

    for _ in range(warmup):
        step()
    # the timed steps, as the metric defines them: K decode steps, each after an
    # untimed write and read of 1 GiB of scratch (flush()), each bracketed by
    # events on the launch stream
    scratch, rsum = flush_buffers()
    torch.cuda.synchronize()
    ev = _events(2 * steps)
    t0 = time.perf_counter()
    for i in range(steps):
        flush(scratch, rsum)
        ev[2 * i].record()
        step()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cold = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]
    # the same steps after the write alone (information: the MALL then holds 256
    # MB of the flush's dirty lines, written back when the step's reads evict them)
    wflush = []
    for i in range(steps):
        scratch.fill_(1)
        e0, e1 = _events(2)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        wflush.append(e0.elapsed_time(e1))

    # warm steps (information only): K steps back to back with the pool partly in
    # the MALL, bracketed by a synchronisation and events, then each by events
    torch.cuda.synchronize()
    e_start, e_end = _events(2)
    e_start.record()
    for _ in range(steps):
        step()
    e_end.record()
    torch.cuda.synchronize()
    warm_total_ms = e_start.elapsed_time(e_end)
    ev = _events(steps + 1)
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    warm_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]

    # the dominant kernel: the tile pass launched back to back (it rewrites the
    # same partials), bracketed by events on its launch stream; the average
    # duration per launch excludes the launch gaps a single pair of events
    # around one launch would add
    tile_ms = []
    for layer in range(wl.shape.n_layers):
        kw = dict(layer=layer, k_params=pool.kp, v_params=pool.vp)
        e0, e1 = _events(2)
        e0.record()
        for _ in range(steps):
            K.paged_decode_attn_phases(wl.shape, plan, qs[layer], pool.k, pool.v, out, ws, K.PHASE_TILES, **kw)
        e1.record()
        K.paged_decode_attn_phases(wl.shape, plan, qs[layer], pool.k, pool.v, out, ws, K.PHASE_COMBINE, **kw)
        torch.cuda.synchronize()
        tile_ms.append(e0.elapsed_time(e1) / steps)

    # read ceiling of this box: a plain read of as many bytes as one tile pass
    # reads, launched back to back like the tile pass; best of a few launch
    # shapes of a grid-stride sweep and of per-workgroup contiguous chunks
    nb = int(a["unique_kv_bytes"]) // 16 * 16
    rbuf = torch.ones(nb, dtype=torch.uint8, device="cuda")
    rout = torch.zeros(4, dtype=torch.int32, device="cuda")
    probe = []
    shapes = [(g, nt, False) for g in (2048, 4096, 8192, 16384) for nt in (False, True)]
    shapes += [(g, True, True) for g in (1024, 2048, 4096)]
    for grid, nt, chunked in shapes:
        wdev.read_probe(rbuf, rout, grid, nt, chunked)
        e0, e1 = _events(2)
        e0.record()
        for _ in range(steps):
            wdev.read_probe(rbuf, rout, grid, nt, chunked)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / steps
        probe.append((nb / (us * 1e-6) / 1e9, grid, nt, us, "chunked" if chunked else "grid-stride"))
    del rbuf
    read_ceiling = max(probe)

    ub = int(a["unique_kv_bytes"]) * wl.shape.n_layers
    if copy_probe:
        # a plain 1 GiB device copy: reference point for the HBM byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(3)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    return dict(wl=wl, tables=T, t_tables=t_tables, wall=wall, warm_total_ms=warm_total_ms, warm_ms=warm_ms, cold_ms=cold,
                wflush_ms=wflush,
                tile_ms=tile_ms, read_ceiling=read_ceiling, unique_bytes=ub, layer_bytes=int(a["unique_kv_bytes"]),
                n_phys=int(a["n_phys"]), n_items=int(a["items"].shape[0]))


def profile_run(cfg, steps, warmup, copy_probe=False):
    """Untimed decode steps for a profiler's counter passes: `warmup` steps, then
    `steps` steps each after the flush of the timed steps (so the tile pass reads
    from HBM, as there), then optionally the plain 1 GiB device copy the HBM
    byte counters are scaled by."""
    import torch

    from shared_paged_kv_amd import _lib as K
    from workload import device as wdev
    from workload import spec

    wl = spec.make(cfg)
    T = K.build_tables(wl.shape, wl.agents)
    a = T.arrays
    plan = K.DevicePlan(T)
    pool = wdev.Pool(wl, a["phys_agent"], a["phys_block"], a["phys_ntok"], a["n_dedup"])
    qs = [wdev.fill_q(wl, layer) for layer in range(wl.shape.n_layers)]
    ws = torch.empty(max(1, K.workspace_bytes(wl.shape, plan)), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.n_agents, wl.shape.n_q_heads, wl.shape.head_dim), dtype=torch.float32, device="cuda")
    scratch, rsum = flush_buffers()

    def step():
        for layer in range(wl.shape.n_layers):
            K.paged_decode_attn(wl.shape, plan, qs[layer], pool.k, pool.v, out, ws, layer=layer,
                                k_params=pool.kp, v_params=pool.vp)

    for _ in range(warmup):
        step()
    for _ in range(steps):
        flush(scratch, rsum)
        step()
    if copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(3)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
    torch.cuda.synchronize()
    return {"profile_only": cfg, "steps": steps, "warmup": warmup, "layers": wl.shape.n_layers,
            "unique_kv_bytes_per_layer": int(a["unique_kv_bytes"])}


def code_text(src: str) -> str:
    """C/C++ source without its comments, whitespace runs collapsed: what a
    comment-only edit leaves unchanged (string and character literals kept)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(cfg: str) -> str:
    """Fingerprint of what sets the tile pass's HBM traffic on a workload: the
    kernel sources (code only: comments do not count) and the work plan the
    library builds for it."""
    import hashlib

    from shared_paged_kv_amd import _lib as K
    from workload import spec

    h = hashlib.sha256()
    for f in ("shared_paged_kv_amd/csrc/hip/decode.hip", "shared_paged_kv_amd/csrc/hip/device_common.h"):
        h.update(code_text(open(os.path.join(ROOT, f)).read()).encode())
    wl = spec.make(cfg)
    a = K.build_tables(wl.shape, wl.agents).arrays
    for k in ("items", "plan_blocks", "cons", "qcons", "mask", "comb_ptr", "comb_rows", "class_items"):
        h.update(np.ascontiguousarray(a[k]).tobytes())
    h.update(np.int64(a["unit_span"]).tobytes())
    return h.hexdigest()[:16]


def measured_traffic(cfg):
    """HBM bytes per tile-pass launch from the committed rocprofv3 counter runs
    (profiles/tile_kernel_<cfg>_hbm_counters.json), or None when there are none
    or the kernel sources or the work plan changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"tile_kernel_{cfg}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_hash") != kernel_source_hash(cfg):
        return None
    return d.get("hbm_bytes_per_launch")


CPU_SAMPLE = """
import json, os, sys, time
sys.path.insert(0, {root!r})
from concurrent.futures import ProcessPoolExecutor
import numpy as np
from workload import rng, spec
from oracle import attention, dedup

wl = spec.make({cfg!r})
sh = wl.shape
t0 = time.perf_counter()
tables = dedup.build_tables(sh.block_tokens, wl.agents)
t_tab = time.perf_counter() - t0
qf = rng.bf16_bits_to_f32(spec.q_bits(wl, 0)).astype(np.float64)
scale = 1.0 / np.sqrt(sh.head_dim)


def work(job):
    # the steps of attention.decode over the tables, timed apart: dense
    # materialisation of the agent's context (the kv heads its q heads read),
    # then its attention
    j, heads = job
    kvh = attention._kv_heads(wl, heads)
    store = attention._Store(wl, 0)
    t0 = time.perf_counter()
    K, V = attention.dense_from_tables(wl, tables, j, store, kvh)
    t1 = time.perf_counter()
    attention.attend(qf[j], K, V, scale)
    return t1 - t0, time.perf_counter() - t1


agents = list(range(min({na}, wl.n_agents)))
nh = min({nh}, sh.n_q_heads)
grp = sh.n_q_heads // sh.n_kv_heads
workers = {workers}
# split every agent's q heads into chunks (whole kv-head groups) so that the
# (agent, chunk) jobs keep every worker busy
n_chunk = max(1, min(-(-nh // grp), -(-workers // len(agents))))
jobs = []
for j in agents:
    hs = list(range(nh))
    gs = sorted({{h // grp for h in hs}})
    for k in range(n_chunk):
        gk = set(gs[len(gs) * k // n_chunk: len(gs) * (k + 1) // n_chunk])
        part = [h for h in hs if h // grp in gk]
        if part:
            jobs.append((j, part))
t0 = time.perf_counter()
with ProcessPoolExecutor(max_workers=workers) as ex:
    res = list(ex.map(work, jobs))
wall = time.perf_counter() - t0
print(json.dumps(dict(seconds=wall, table_build=t_tab, materialise=sum(r[0] for r in res),
                      attention=sum(r[1] for r in res), heads=nh, agents=len(agents), workers=workers,
                      jobs=len(jobs), os_cpu_count=os.cpu_count())))
"""

# worker processes of the CPU baseline: the host's cores, at most the 16 a
# one-GPU share of the machine has
CPU_WORKERS = max(1, min(16, os.cpu_count() or 1))


def cpu_baseline(cfg, n_agents, n_heads, workers=None):
    """The oracle as it stands on n_agents agents x n_heads q heads of layer 0 of
    the workload: its dedup tables built once, then every (agent, head chunk)
    materialised and attended in a pool of `workers` processes, one BLAS thread
    each.  Returns the wall time of the pool and the CPU seconds per phase."""
    workers = CPU_WORKERS if workers is None else workers
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    code = CPU_SAMPLE.format(root=ROOT, cfg=cfg, nh=n_heads, na=n_agents, workers=workers)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=900)
    if r.returncode:
        raise RuntimeError(r.stderr[-2000:])
    return json.loads(r.stdout.strip().splitlines()[-1])


def lifecycle_run(cfg, steps, warmup):
    """Device cost of one decode step's appends (include/kvpool_lifecycle.h):
    one token for every agent of the config, which copies every shared last
    block with room (copy-on-write) and writes each token in its block's frame,
    in every layer.  The pool tensors are allocated at their full size but not
    filled (the copy's cost does not depend on the bytes); the same operations
    are re-run each step (copies and writes are idempotent)."""
    import torch

    from shared_paged_kv_amd import _lib as K
    from workload import spec

    wl = spec.make(cfg)
    sh = wl.shape
    T = K.build_tables(sh, wl.agents)
    cap = T.n_phys + 2 * wl.n_agents
    bp = K.BlockPool(T, sh, cap)
    t0 = time.perf_counter()
    cp, wr = bp.append(list(range(wl.n_agents)))
    t_host = time.perf_counter() - t0
    shape5 = (sh.n_layers, cap, sh.n_kv_heads, sh.block_tokens, sh.head_dim)
    kp = torch.empty(shape5, dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    rows = (sh.n_layers, wl.n_agents, sh.n_kv_heads, sh.head_dim)
    kn = torch.randn(rows, device="cuda").to(torch.bfloat16)
    vn = torch.randn(rows, device="cuda").to(torch.bfloat16)
    c = torch.from_numpy(cp.reshape(-1).copy()).cuda() if len(cp) else None
    w = torch.from_numpy(wr.reshape(-1).copy()).cuda() if len(wr) else None

    def step():
        K.kv_append(sh, kp, vp, cap, c, w, kn, vn, wl.n_agents)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / steps
    # algorithmic HBM bytes: every distinct copy source read once, every copy
    # written, every new row read and written to its slot (K and V, all layers)
    block_layer = sh.n_kv_heads * sh.block_tokens * sh.head_dim * 2 * 2
    row_layer = sh.n_kv_heads * sh.head_dim * 2 * 2
    n_src = len(set(int(x) for x in cp[:, 0])) if len(cp) else 0
    moved = (n_src + len(cp)) * sh.n_layers * block_layer + len(wr) * sh.n_layers * row_layer * 2
    return {"metric": "kv_append (copy-on-write + token writes) HBM GB/s", "value": round(moved / us / 1e3, 1),
            "unit": "GB/s", "peak": HBM_PEAK_GBPS, "frac": round(moved / us / 1e3 / HBM_PEAK_GBPS, 4),
            "us_per_step": round(us, 2), "bytes_per_step": moved, "copies": int(len(cp)), "copy_sources": n_src,
            "writes": int(len(wr)),
            "host_append_ms": round(t_host * 1000.0, 3), "steps": steps,
            "config": {"workload": f"{cfg}: {wl.n_agents} agents, {sh.n_layers} layer(s), one appended token each"}}


def mirror_run(cfg, steps, warmup):
    """Device cost of the master/mirror steps (include/kvpool_mirror.h) over a
    whole round: every agent's context restored into paged buffers, fused (one
    pass: delta or master block, re-rotated, written once) and unfused (copy
    every master block, overwrite the delta blocks, re-rotate every K row);
    then the diff scan of every agent's blocks (in the master's frame) against
    its master blocks, threshold 0."""
    import torch

    from shared_paged_kv_amd import _lib as K
    from workload import device as wdev
    from workload import spec

    wl = spec.make(cfg)
    sh = wl.shape
    T = K.build_tables(sh, wl.agents)
    a = T.arrays
    pool = wdev.Pool(wl, a["phys_agent"], a["phys_block"], a["phys_ntok"], a["n_dedup"])
    P = pool.capacity
    fused = K.restore_list(T, list(range(wl.n_agents)))   # grouped by source
    n = len(fused)
    by_dst = fused[np.argsort(fused[:, 3], kind="stable")]
    nb = a["n_blocks"]
    master_id = np.concatenate([a["block_table"][j, :nb[j]] for j in range(wl.n_agents)])
    delta_id = np.concatenate([a["delta_table"][j, :nb[j]] for j in range(wl.n_agents)])
    dst = np.arange(n, dtype=np.int32)
    nt, shift = by_dst[:, 2], by_dst[:, 1]
    zero = np.zeros(n, np.int32)
    master = np.stack([master_id, zero, nt, dst], 1)
    master = master[np.lexsort((master[:, 3], master[:, 2], master[:, 0]))]   # grouped by source too
    has = delta_id >= 0
    delta = np.stack([delta_id[has], zero[has], nt[has], dst[has]], 1)
    cand = fused.copy()
    cand[:, 1] = 0
    pairs = np.stack([master_id, dst, nt], 1)
    pairs = pairs[np.argsort(pairs[:, 0], kind="stable")]                      # adjacent masters
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.int32).reshape(-1)).cuda()
    fused_d, master_d, delta_d, pairs_d = dev(fused), dev(master), dev(delta), dev(pairs)
    shp = (sh.n_layers, n, sh.n_kv_heads, sh.block_tokens, sh.head_dim)
    dk = torch.empty(shp, dtype=torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    # the re-rotation pass takes a block as one row of Hkv * B heads (one shift each)
    rows = dk.view(-1, sh.n_kv_heads * sh.block_tokens, sh.head_dim)
    row_shift = dev(np.tile(shift, sh.n_layers))
    flags = torch.empty(n, dtype=torch.int32, device="cuda")

    def fused_step():
        K.kv_restore(sh, pool.k, pool.v, P, fused_d, dk, dv, n)

    def three_pass_step():
        K.kv_restore(sh, pool.k, pool.v, P, master_d, dk, dv, n)
        K.kv_restore(sh, pool.k, pool.v, P, delta_d, dk, dv, n)
        K.kv_rerotate(rows, row_shift, sh.rope_theta, out=rows)

    def diff_step():
        K.kv_diff_blocks(sh, pool.k, pool.v, P, cand_k, cand_v, n, pairs_d, 0.0, flags)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = _events(2)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / steps

    us_fused = timed(fused_step)
    us_three = timed(three_pass_step)
    # candidates: every agent's blocks in the master's stored frame
    K.kv_restore(sh, pool.k, pool.v, P, dev(cand), dk, dv, n)
    cand_k, cand_v = dk, dv
    us_diff = timed(diff_step)
    n_diff = int(flags.sum().item())
    n_delta = len(delta)
    block_layer = sh.n_kv_heads * sh.block_tokens * sh.head_dim * 2 * 2   # K and V
    L = sh.n_layers
    # restore: every distinct source block read once, every destination written
    restore_bytes = (len(set(fused[:, 0].tolist())) + n) * L * block_layer
    # diff: every candidate that matches its master is read whole, and each
    # distinct master once (a differing pair may stop at its first difference)
    diff_bytes = (n - n_diff + len(set(pairs[:, 0].tolist()))) * L * block_layer
    gb = lambda b, us: round(b / us / 1e3, 1)
    return {"metric": "fused mirror restore HBM GB/s", "value": gb(restore_bytes, us_fused), "unit": "GB/s",
            "peak": HBM_PEAK_GBPS, "frac": round(restore_bytes / us_fused / 1e3 / HBM_PEAK_GBPS, 4),
            "us_fused": round(us_fused, 1), "us_three_pass": round(us_three, 1),
            "three_pass_over_fused": round(us_three / us_fused, 3), "restore_bytes": restore_bytes,
            "diff": {"us": round(us_diff, 1), "GBps": gb(diff_bytes, us_diff),
                     "frac": round(diff_bytes / us_diff / 1e3 / HBM_PEAK_GBPS, 4), "bytes": diff_bytes,
                     "blocks": n, "flagged": n_diff, "deltas": n_delta},
            "steps": steps,
            "config": {"workload": f"{cfg}: {wl.n_agents} agents, {n} logical blocks, {n_delta} deltas, "
                                   f"{sh.n_layers} layer(s)"}}


def persist_run(cfg, steps, warmup, layers):
    """Persistent Q4 pool (include/kvpool_persist.h) on the config's agents with
    a `layers`-layer cache: one agent's blocks saved to a safetensors file
    (device->host gather, file write), read back (file read from the page
    cache), and loaded into the pool (host->device copies, all layers); then the
    load overlapped with the round's decode (one step = the decode attention of
    every layer) on a second stream."""
    import tempfile

    import torch

    from shared_paged_kv_amd import _lib as K
    from workload import device as wdev
    from workload import spec

    wl = spec.make(cfg)
    sh = wl.shape
    if sh.kv_dtype != spec.Q4G64:
        raise SystemExit(f"--persist stores Q4 pools; the {cfg} config is not one (use --config q4)")
    sh.n_layers = layers
    T = K.build_tables(sh, wl.agents)
    a = T.arrays
    pool = wdev.Pool(wl, a["phys_agent"], a["phys_block"], a["phys_ntok"], a["n_dedup"])
    P = pool.capacity
    tensors = (pool.k, pool.v, pool.kp, pool.vp)
    plan = K.DevicePlan(T)
    ws = torch.empty(max(1, K.workspace_bytes(sh, plan)), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.n_agents, sh.n_q_heads, sh.head_dim), dtype=torch.float32, device="cuda")
    qs = [wdev.fill_q(wl, l) for l in range(layers)]
    j = 0
    ids = [int(x) for x in a["block_table"][j, :a["n_blocks"][j]]]
    nb = K.q4_image_bytes(sh, len(ids))
    img = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
    path = os.path.join(tempfile.mkdtemp(prefix="kvpool_q4_"), "agent0.safetensors")
    ntok = a["phys_ntok"][ids]

    def clock(fn, reps):
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        return (time.perf_counter() - t0) / reps

    def save():
        K.kv_q4_gather(sh, *tensors, P, ids, img)
        torch.cuda.synchronize()
        K.q4_save_file(sh, path, "agent-0", img, ntok)

    def read():
        K.q4_load_file(sh, path, "agent-0", img)

    side = torch.cuda.Stream()

    def load_on(stream):
        with torch.cuda.stream(stream):
            K.kv_q4_scatter(sh, img, *tensors, P, ids)

    def decode_step():
        for l in range(layers):
            K.paged_decode_attn(sh, plan, qs[l], pool.k, pool.v, out, ws, layer=l, k_params=pool.kp,
                                v_params=pool.vp)

    t_save = clock(save, 3)
    t_read = clock(read, 3)
    for _ in range(warmup):
        decode_step()
        load_on(side)
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    e = _events(6)
    # load alone (side stream), decode alone (main stream), then both together
    e[0].record(side)
    for _ in range(steps):
        load_on(side)
    e[1].record(side)
    torch.cuda.synchronize()
    e[2].record()
    for _ in range(steps):
        decode_step()
    e[3].record()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    start.record()
    side.wait_event(start)
    for _ in range(steps):
        load_on(side)
    for _ in range(steps):
        decode_step()
    e[4].record()
    e[5].record(side)
    torch.cuda.synchronize()
    t_load = e[0].elapsed_time(e[1]) / steps
    t_dec = e[2].elapsed_time(e[3]) / steps
    t_both = max(start.elapsed_time(e[4]), start.elapsed_time(e[5])) / steps
    hidden = (t_load + t_dec - t_both) / min(t_load, t_dec)
    os.remove(path)
    gbs = lambda b, ms: round(b / ms / 1e6, 2)
    return {"metric": "Q4 pool reload (host->device) GB/s", "value": gbs(nb, t_load), "unit": "GB/s",
            "agent_bytes": nb, "blocks": len(ids), "layers": layers,
            "save_ms": round(t_save * 1e3, 2), "save_GBps": gbs(nb, t_save * 1e3),
            "file_read_ms": round(t_read * 1e3, 2), "file_read_GBps": gbs(nb, t_read * 1e3),
            "load_ms": round(t_load, 3), "decode_step_ms": round(t_dec, 3), "both_ms": round(t_both, 3),
            "overlap": round(hidden, 3),
            "decode_slowdown": round(start.elapsed_time(e[4]) / steps / t_dec, 3), "steps": steps,
            "config": {"workload": f"{cfg}: agent 0 of {wl.n_agents}, {len(ids)} blocks x {layers} layers "
                                   f"({nb / 1e6:.1f} MB Q4); decode step = {layers} layers x {wl.n_agents} agents"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=None, help="workload (default: inms; q4 with --persist)")
    ap.add_argument("--cpu-agents", type=int, default=None,
                    help="agents of the CPU baseline sample (default: all; 32 on rounds of more than 64)")
    ap.add_argument("--cpu-heads", type=int, default=1 << 30, help="q heads per agent of the CPU sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--lifecycle", action="store_true",
                    help="measure one decode step's appends (copy-on-write + token writes) instead")
    ap.add_argument("--persist", action="store_true",
                    help="measure the Q4 pool save / file read / reload, and the reload overlapped with decode")
    ap.add_argument("--layers", type=int, default=32, help="cache layers for --persist")
    ap.add_argument("--profile-only", action="store_true",
                    help="only run untimed decode steps (each after a 1 GiB write) for rocprofv3 counter passes")
    ap.add_argument("--mirror", action="store_true",
                    help="measure the master/mirror restore (fused and three-pass) and diff scan instead")
    args = ap.parse_args()
    if args.config is None:
        args.config = "q4" if args.persist else "inms"
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the decode path has no multi-GPU leg); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if args.lifecycle:
        print(json.dumps(lifecycle_run(args.config, args.steps, args.warmup)), flush=True)
        return
    if args.mirror:
        print(json.dumps(mirror_run(args.config, args.steps, args.warmup)), flush=True)
        return
    if args.persist:
        print(json.dumps(persist_run(args.config, args.steps, args.warmup, args.layers)), flush=True)
        return
    if args.profile_only:
        print(json.dumps(profile_run(args.config, args.steps, args.warmup, args.copy_probe)), flush=True)
        return

    r = gpu_run(args.config, args.steps, args.warmup, args.copy_probe)
    wl = r["wl"]
    pct = lambda x, q: round(float(np.percentile(x, q)) * 1000, 2)
    ms = float(np.median(r["cold_ms"]))
    value = wl.n_agents / (ms / 1000.0)
    gbps = r["unique_bytes"] / (ms / 1000.0) / 1e9
    warm_ms = r["warm_total_ms"] / args.steps
    tile_us = float(np.mean(r["tile_ms"])) * 1000.0
    tile_gbps = r["layer_bytes"] / (tile_us * 1e-6) / 1e9
    rc = r["read_ceiling"]
    res = {
        "metric": "decode-attn agent-tokens/s (effective unique-KV HBM GB/s vs peak alongside)",
        "value": round(value, 1),
        "unit": "agent-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",  # the products run in bf16 (Q4 codes are exact in it), accumulation in fp32
        "data": "synthetic (seeded Philox draws, shapes of the pages' workloads)",
        "config": {
            "workload": f"{args.config}: {wl.n_agents} agents x {wl.context_len(0)} tokens, "
                        f"Hq {wl.shape.n_q_heads} / Hkv {wl.shape.n_kv_heads} x {wl.shape.head_dim}, "
                        f"block {wl.shape.block_tokens}, {wl.shape.n_layers} layer(s)",
            "kv_storage": "bf16" if wl.shape.kv_dtype == 0 else "q4g64",
            "n_agents": wl.n_agents, "physical_blocks": r["n_phys"], "work_items": r["n_items"],
            "unique_kv_bytes_per_step": r["unique_bytes"],
        },
        "timing": "value and ms_per_step: median of the K timed steps, each a decode step over every layer "
                  "after an untimed write and read of 1 GiB (L2 and MALL evicted, MALL left clean), events on "
                  "the launch stream",
        "effective_GBps": round(gbps, 1),
        "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "step_us": {"median": round(ms * 1000, 2), "p10": pct(r["cold_ms"], 10), "p90": pct(r["cold_ms"], 90)},
        "write_flush_step_us": {"note": "the same steps after the 1 GiB write alone (the MALL then holds the "
                                        "write's dirty lines, written back during the step); information only",
                                "median": round(float(np.median(r["wflush_ms"])) * 1000, 2),
                                "p10": pct(r["wflush_ms"], 10), "p90": pct(r["wflush_ms"], 90)},
        "timed_wall_s": round(r["wall"], 4),
        "warm": {"note": "K steps back to back, no flush (pool partly resident in the MALL); information only",
                 "ms_per_step": round(warm_ms, 5), "value": round(wl.n_agents / (warm_ms / 1000.0), 1),
                 "effective_GBps": round(r["unique_bytes"] / (warm_ms / 1000.0) / 1e9, 1),
                 "step_us": {"median": round(float(np.median(r["warm_ms"])) * 1000, 2),
                             "p10": pct(r["warm_ms"], 10), "p90": pct(r["warm_ms"], 90)}},
        "table_build_s": round(r["t_tables"], 4),
        "roofline": {"bound": "hbm", "kernel": "tile_kernel (tile pass)", "achieved": round(tile_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(tile_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(args.config),
                     "algorithmic_bytes_per_launch": r["layer_bytes"], "avg_launch_us": round(tile_us, 2),
                     "read_ceiling": {"kernel": "plain 16-byte read of the same byte count (best of a "
                                                "grid-stride sweep and per-workgroup contiguous chunks)",
                                      "GBps": round(rc[0], 1), "frac": round(tile_gbps / rc[0], 4),
                                      "pattern": rc[4], "grid": rc[1], "nontemporal": rc[2],
                                      "avg_launch_us": round(rc[3], 2)}},
    }
    if not args.no_cpu:
        na = args.cpu_agents if args.cpu_agents is not None else (32 if wl.n_agents > 64 else wl.n_agents)
        c = cpu_baseline(args.config, na, args.cpu_heads)
        # one layer is timed; a step covers every layer of the config
        per_step_s = c["seconds"] * wl.shape.n_layers
        agent_steps = c["agents"] * c["heads"] / wl.shape.n_q_heads
        res["cpu_baseline"] = {"value": round(agent_steps / per_step_s, 4),
                               "unit": "agent-tokens/s", "cores": c["workers"], "kind": "oracle",
                               "sample": f"{c['agents']} of {wl.n_agents} agents x {c['heads']} of "
                                         f"{wl.shape.n_q_heads} q heads, layer 0"
                                         + (f" (x{wl.shape.n_layers} layers, extrapolated)" if wl.shape.n_layers > 1
                                            else "")
                                         + f", float64 oracle: dense materialisation through its tables + "
                                         f"attention, {c['jobs']} (agent, head-chunk) jobs over {c['workers']} "
                                         f"worker processes of one BLAS thread each ({c['seconds']:.1f} s wall); "
                                         f"table build of the whole workload apart",
                               "os_cpu_count": c["os_cpu_count"], "blas_threads_per_worker": 1,
                               "split_s": {"table_build": round(c["table_build"], 3),
                                           "materialise_cpu_s": round(c["materialise"], 3),
                                           "attention_cpu_s": round(c["attention"], 3)}}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
