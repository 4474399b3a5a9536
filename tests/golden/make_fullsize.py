"""Writes the oracle's decode outputs for the full-size workloads to
tests/golden/fullsize_<name>.npz, for the GPU parity tests to compare every
output of the full-size runs against.

Calls only ``oracle`` (dense per-agent materialisation and float64 attention)
and the seeded workload generator; nothing here runs on or reads from the GPU
path.  The oracle is the plain definition, so the whole set takes minutes of
CPU; the agents are spread over worker processes, each running the oracle on a
contiguous share of them (shared content is regenerated per worker, which
changes nothing in the result).

Outputs are stored as float32 (their rounding, ~1e-9 here, is far below every
tolerance) together with the workload fingerprint, the agents and the layers.

Usage:  python -m tests.golden.make_fullsize [name ...]    (default: all four)
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

# scale round: the layers compared, and 32 agents -- both ends, one in the middle,
# and three from each of the ten equal consumer groups the shared segments are
# split into (25 consumers of 5 q heads each make a 125-row group)
SCALE_LAYERS = (0, 47)
SCALE_AGENTS = sorted({0, 137, 249} | {25 * k + o for k in range(10) for o in (3, 14, 24)})


def selection(name: str):
    """(agents, layers) whose outputs are stored for workload `name`."""
    from workload import spec
    if name == "scale":
        return list(SCALE_AGENTS), list(SCALE_LAYERS)
    wl = spec.make(name)
    return list(range(wl.n_agents)), [0]


def path(name: str) -> str:
    return os.path.join(HERE, f"fullsize_{name}.npz")


def load(name: str, wl=None):
    """(out [layers][agents][Hq][d] float64, agents, layers) stored for `name`;
    raises if the file's fingerprint is not the workload's (the generator changed:
    run this script again)."""
    from workload import spec
    wl = spec.make(name) if wl is None else wl
    d = np.load(path(name), allow_pickle=False)
    fp = str(d["fingerprint"])
    if fp != spec.fingerprint(wl):
        raise RuntimeError(f"{path(name)} was written for another {name} workload (fingerprint {fp[:16]}); "
                           f"regenerate it with python -m tests.golden.make_fullsize {name}")
    return d["out"].astype(np.float64), [int(x) for x in d["agents"]], [int(x) for x in d["layers"]]


def _work(args):
    name, layer, agents = args
    os.environ.setdefault("OPENBLAS_NUM_THREADS", "1")
    from oracle import attention
    from workload import spec
    wl = spec.make(name)
    return attention.decode(wl, layer, agents=agents)


def make(name: str, procs: int) -> None:
    from concurrent.futures import ProcessPoolExecutor
    from workload import spec
    wl = spec.make(name)
    agents, layers = selection(name)
    t0 = time.time()
    nch = min(len(agents), procs * 2)
    chunks = [agents[len(agents) * k // nch: len(agents) * (k + 1) // nch] for k in range(nch)]
    jobs = [(name, layer, ch) for layer in layers for ch in chunks if ch]
    with ProcessPoolExecutor(max_workers=procs) as ex:
        res = list(ex.map(_work, jobs))
    out = np.zeros((len(layers), len(agents), wl.shape.n_q_heads, wl.shape.head_dim), np.float32)
    k = 0
    for li in range(len(layers)):
        a0 = 0
        for ch in chunks:
            if not ch:
                continue
            out[li, a0:a0 + len(ch)] = res[k]
            a0 += len(ch)
            k += 1
    np.savez(path(name), out=out, agents=np.array(agents, np.int32), layers=np.array(layers, np.int32),
             fingerprint=np.array(spec.fingerprint(wl)))
    print(f"{name}: {len(layers)} layer(s) x {len(agents)} agents in {time.time() - t0:.0f} s -> {path(name)}",
          flush=True)


def main(argv):
    names = argv or ["inms", "q4", "tokendance", "scale"]
    procs = os.cpu_count() or 1
    for n in names:
        make(n, procs)


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
    main(sys.argv[1:])
