"""paged_decode_attn_noalloc (include/kvpool.h): the decode on the library's own
per-device scratch array, for callers that cannot allocate device memory,
against paged_decode_attn with a caller-provided workspace -- several calls in a
row on one device, each on a smaller round than the one before, so that every
call finds the previous call's contents in the shared array -- and its size
limit."""
import ctypes as C

import numpy as np
import pytest

from oracle import attention
from shared_paged_kv_amd import _lib as K
from workload import spec

from .gpu_util import Case, log
from .tolerances import ATOL, gate


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_point():
    import torch
    # largest first: TokenDance (shifted consumers, wide items, ~18 MB of
    # workspace), then a small round with shifts and deltas, then a Q4 round
    for name in ["tokendance", "small_round", "tiny_q4"]:
        wl = spec.make(name)
        log("case", name)
        c = Case(wl)
        need = K.workspace_bytes(wl.shape, c.plan)
        assert 0 < need <= K.NOALLOC_SCRATCH_BYTES
        q = c.q(0)
        ref = c.run(0, q=q)
        out = torch.full_like(c.out, float("nan"))
        for _ in range(2):
            K.paged_decode_attn_noalloc(wl.shape, c.plan, q, c.pool.k, c.pool.v, out, layer=0,
                                        k_params=c.pool.kp, v_params=c.pool.vp)
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            # the same kernels in the same order: bit-identical outputs
            assert np.array_equal(got, ref), f"{name}: max-abs {np.abs(got - ref).max():.3e}"
        if name != "tokendance":
            exp = attention.decode(wl, 0)
            L = max(wl.context_len(j) for j in range(wl.n_agents))
            err = float(np.abs(got - exp).max())
            log(f"  {name}: max-abs vs oracle {err:.3e}")
            assert err <= ATOL and err <= gate(exp, L)
        del c


def test_noalloc_rejects_plans_beyond_its_scratch():
    """A plan whose workspace exceeds KVP_NOALLOC_SCRATCH_BYTES is refused with
    KVP_EWORKSPACE before anything touches the device (so this runs without a
    GPU: the plan's pointers are never read)."""
    n = 520   # agents of one private 16-token block each: 520 partial rows x 512 kv heads x 128 floats
    sh = spec.Shape(1, 512, 512, 128, 16, spec.BF16, 1e4)
    g = np.random.default_rng(7)
    agents = [spec.Agent([spec.Span(spec.PRIVATE, 0, spec.PREFIX, g.integers(1, 1 << 30, 16).astype(np.int32))])
              for _ in range(n)]
    T = K.build_tables(sh, agents)
    a = T.arrays
    p = K.kvp_plan_dev()
    p.n_agents, p.n_phys, p.n_items = a["n_agents"], a["n_phys"], int(a["items"].shape[0])
    p.n_qcons, p.n_qcons_shifted, p.n_part_rows = int(a["n_qcons"]), int(a["n_qcons_shifted"]), int(a["n_part_rows"])
    for i in range(6):
        p.class_items[i] = int(a["class_items"][i])
    p.unit_span = int(a["unit_span"])
    for k in K.PLAN_ARRAYS:
        setattr(p, k, 0x1000)   # never dereferenced: the size check comes first
    need = C.c_size_t()
    cs = K.make_shape(sh)
    assert K.lib().paged_decode_attn_workspace_bytes(C.byref(cs), C.byref(p), C.byref(need)) == K.KVP_OK
    assert need.value > K.NOALLOC_SCRATCH_BYTES
    fake = C.c_void_p(0x1000)
    rc = K.lib().paged_decode_attn_noalloc(C.byref(cs), C.byref(p), fake, fake, fake, None, None, 0, 0.088,
                                           fake, None)
    assert rc == K.KVP_EWORKSPACE
    msg = K.lib().kvpool_last_error().decode()
    assert str(need.value) in msg and str(K.NOALLOC_SCRATCH_BYTES) in msg
