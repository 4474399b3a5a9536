"""The checked build (shared_paged_kv_amd/libkvpool_checked.so: bounds checks on
the table indices inside the kernels) on the device, in a child process that
loads it in place of the ordinary library:

* decode rounds that reach every kernel path (the small configs, seeded random
  rounds over head dims, block sizes, dtypes, GQA groups and the XCD-pinned
  mapping, and the full TokenDance round with its wide items) run with the
  error word left at 0, and their outputs match the oracle;
* a plan whose device copy is corrupted after the host's checks -- a physical
  block id, a consumer entry, a combine entry, an item's block range, each one
  past the end of what it indexes -- is caught by the kernels' own checks: the
  error word gets the matching bit, and the workgroups that see it return
  before touching a pool (every kernel exits normally).  The plan is restored
  after each case and the next clean run matches the oracle again."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import json, sys
sys.path.insert(0, {root!r})
import numpy as np
import torch
from oracle import attention
from shared_paged_kv_amd import _lib as K
from tests.gpu_util import Case
from tests.test_gpu_random import random_round
from tests.tolerances import ATOL, gate
from workload import spec

assert K.device_checks_enabled(), K.LIB_PATH
res = {{"clean": [], "corrupt": {{}}}}

def check(name, wl, c):
    got = c.run(0)
    ref = attention.decode(wl, 0)
    err = float(np.abs(got - ref).max())
    ok = bool(np.isfinite(got).all()) and err <= ATOL and all(
        float(np.abs(got[j] - ref[j]).max()) <= gate(ref[j], wl.context_len(j)) for j in range(wl.n_agents))
    return [name, err, ok, K.take_device_errors()]

cases = [(n, spec.make(n)) for n in ("tiny", "tiny_seg", "tiny_q4", "small_round")]
cases += [("random%d" % s, random_round(s)) for s in range(12)]
cases += [("random%d_h%d_%d" % (s, hq, hkv), random_round(s, heads=(hq, hkv))) for s, (hq, hkv) in
          ((20, (8, 8)), (21, (16, 8)), (22, (32, 16)), (23, (40, 8)))]
cases += [("random%d_q4" % s, random_round(s, q4=True)) for s in (30, 31)]
for name, wl in cases:
    print("case", name, flush=True)
    res["clean"].append(check(name, wl, Case(wl)))
    torch.cuda.empty_cache()

# corrupted device copies of small_round's plan, restored after each
wl = spec.make("small_round")
c = Case(wl)
a = c.T.arrays
t = c.plan.tensors
def corrupt(name, tensor, index, value, bit):
    old = int(tensor[index])
    tensor[index] = value
    c.run(0)
    e = K.take_device_errors()
    tensor[index] = old
    res["corrupt"][name] = [e, bit]
    print("corrupt", name, e, flush=True)
corrupt("block id", t["plan_blocks"], len(a["plan_blocks"]) // 2, int(a["n_phys"]), 2)
corrupt("consumer", t["cons"], len(a["cons"]) - 1, int(a["n_qcons"]), 4)
corrupt("combine entry", t["comb_rows"], len(a["comb_rows"]) // 2, int(a["n_part_rows"]), 8)
corrupt("item blocks", t["items"], 1, len(a["plan_blocks"]) + 1, 1)   # items[0].blk_end
res["clean"].append(check("small_round restored", wl, c))
del c
torch.cuda.empty_cache()

wl = spec.make("tokendance")
print("case tokendance", flush=True)
res["clean"].append(check("tokendance", wl, Case(wl)))
print(json.dumps(res), flush=True)
"""


def test_checked_build_on_device():
    lib = os.path.join(ROOT, "shared_paged_kv_amd", "libkvpool_checked.so")
    assert os.path.exists(lib), "build the library first (python -m shared_paged_kv_amd.build)"
    env = dict(os.environ, KVPOOL_LIB=lib)
    r = subprocess.run([sys.executable, "-u", "-c", CHILD.format(root=ROOT)], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    print(r.stdout[-4000:], r.stderr[-4000:])
    assert r.returncode == 0
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert len(res["clean"]) >= 20
    for name, err, ok, dev_err in res["clean"]:
        assert ok, (name, err)
        assert dev_err == 0, (name, dev_err)
    assert set(res["corrupt"]) == {"block id", "consumer", "combine entry", "item blocks"}
    for name, (got, bit) in res["corrupt"].items():
        assert got & bit, (name, got)
