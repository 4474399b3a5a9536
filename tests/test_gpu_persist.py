"""Persistent Q4 pool on the GPU through the C ABI: kv_q4_gather / kv_q4_scatter
byte for byte against the oracle's image and scatter; every agent's blocks
saved to its own file, the pool wiped, the files reloaded (each under its agent
namespace) and the decode bit-identical to the decode before; a reload on a
second stream while decodes run on the first."""
import numpy as np
import pytest

from oracle import persist as ops
from shared_paged_kv_amd import _lib as K
from workload import device as wdev
from workload import spec

from .gpu_util import log

pytestmark = pytest.mark.gpu


def _tiny_q4_3_layers():
    wl = spec.make("tiny_q4")
    wl.shape.n_layers = 3
    return wl


_CASES = {"tiny_q4": lambda: spec.make("tiny_q4"), "tiny_q4_3_layers": _tiny_q4_3_layers,
          "q4": lambda: spec.make("q4")}


class Setup:
    def __init__(self, wl):
        import torch
        self.wl = wl
        sh = wl.shape
        self.T = K.build_tables(sh, wl.agents)
        a = self.a = self.T.arrays
        self.pool = wdev.Pool(wl, a["phys_agent"], a["phys_block"], a["phys_ntok"], a["n_dedup"])
        self.P = self.pool.capacity
        self.plan = K.DevicePlan(self.T)
        self.ws = torch.empty(max(1, K.workspace_bytes(sh, self.plan)), dtype=torch.uint8, device="cuda")
        self.out = torch.empty((wl.n_agents, sh.n_q_heads, sh.head_dim), dtype=torch.float32, device="cuda")

    @property
    def tensors(self):
        p = self.pool
        return p.k, p.v, p.kp, p.vp

    def host(self):
        import torch
        k, v, kp, vp = self.tensors
        return [k.cpu().numpy(), v.cpu().numpy(), kp.view(torch.int16).cpu().numpy().view(np.float16),
                vp.view(torch.int16).cpu().numpy().view(np.float16)]

    def decode(self, layer=0):
        import torch
        K.paged_decode_attn(self.wl.shape, self.plan, wdev.fill_q(self.wl, layer), self.pool.k, self.pool.v,
                            self.out, self.ws, layer=layer, k_params=self.pool.kp, v_params=self.pool.vp)
        torch.cuda.synchronize()
        return self.out.clone()

    def agent_ids(self, j):
        m = int(self.a["n_blocks"][j])
        return [int(x) for x in self.a["block_table"][j, :m]]


def _pinned(n):
    import torch
    return torch.empty(max(1, n), dtype=torch.uint8, pin_memory=True)


def _as_bytes(img, n):
    return img.numpy()[:n].tobytes()


@pytest.mark.parametrize("name", ["tiny_q4", "tiny_q4_3_layers"])
def test_gather_and_scatter_bytes(name):
    import torch
    wl = _CASES[name]()
    sh = wl.shape
    s = Setup(wl)
    P = s.P
    g = np.random.default_rng(8)
    cases = [list(range(P)), list(range(P))[::-1], [0], [P - 1, 0, 1, 2, P // 2, P // 2 + 1],
             [int(x) for x in g.permutation(P)[: P // 2]]]
    before = s.host()
    for ids in cases:
        n = len(ids)
        nb = K.q4_image_bytes(sh, n)
        img = _pinned(nb)
        K.kv_q4_gather(sh, *s.tensors, P, ids, img)
        torch.cuda.synchronize()
        assert _as_bytes(img, nb) == ops.q4_image(*before, ids)
    log(f"case {name}: gather of {len(cases)} id lists bit-exact")
    # scatter random bytes (ids without repeats), then the pool against the oracle
    for ids in cases[2:]:
        n = len(ids)
        nb = K.q4_image_bytes(sh, n)
        img = _pinned(nb)
        img.numpy()[:] = g.integers(0, 256, nb, dtype=np.uint8)
        cur = s.host()
        K.kv_q4_scatter(sh, img, *s.tensors, P, ids)
        torch.cuda.synchronize()
        want = ops.scatter(cur, _as_bytes(img, nb), ids)
        for got, w in zip(s.host(), want):
            assert np.array_equal(got.view(np.uint8), w.view(np.uint8))
    log(f"case {name}: scatter bit-exact")


@pytest.mark.parametrize("name", ["tiny_q4", "tiny_q4_3_layers", "q4"])
def test_save_wipe_reload_decode(name, tmp_path):
    import torch
    wl = _CASES[name]()
    sh = wl.shape
    s = Setup(wl)
    layers = sorted({0, sh.n_layers - 1})
    ref = {layer: s.decode(layer) for layer in layers}
    before = s.host()
    for j in range(wl.n_agents):
        ids = s.agent_ids(j)
        nb = K.q4_image_bytes(sh, len(ids))
        img = _pinned(nb)
        K.kv_q4_gather(sh, *s.tensors, s.P, ids, img)
        torch.cuda.synchronize()
        K.q4_save_file(sh, tmp_path / f"agent{j}.safetensors", f"agent-{j}", img, s.a["phys_ntok"][ids])
    for t in s.tensors:
        t.zero_()
    torch.cuda.synchronize()
    for j in range(wl.n_agents):
        ids = s.agent_ids(j)
        img = _pinned(K.q4_image_bytes(sh, len(ids)))
        n, ntok = K.q4_load_file(sh, tmp_path / f"agent{j}.safetensors", f"agent-{j}", img)
        assert n == len(ids) and np.array_equal(ntok, s.a["phys_ntok"][ids])
        with pytest.raises(K.KvpError):
            K.q4_load_file(sh, tmp_path / f"agent{j}.safetensors", f"agent-{j + 1}", img)
        K.kv_q4_scatter(sh, img, *s.tensors, s.P, ids)
        torch.cuda.synchronize()   # the image is reused by the next agent
    for got, w in zip(s.host(), before):
        assert np.array_equal(got.view(np.uint8), w.view(np.uint8))
    for layer in layers:
        assert torch.equal(s.decode(layer), ref[layer])
    log(f"case {name}: {wl.n_agents} agents saved, wiped, reloaded; decode bit-identical on layers {layers}")


def test_reload_on_a_second_stream_during_decode(tmp_path):
    import torch
    wl = spec.make("q4")
    sh = wl.shape
    s = Setup(wl)
    ref = s.decode(0)
    j = 3
    ids = s.agent_ids(j)
    nb = K.q4_image_bytes(sh, len(ids))
    img = _pinned(nb)
    K.kv_q4_gather(sh, *s.tensors, s.P, ids, img)
    torch.cuda.synchronize()
    want = s.host()
    # wipe the agent's blocks, then reload them on a side stream while the main
    # stream decodes (those decodes read the wiped blocks: only the last one,
    # after the join, is checked)
    for t in s.tensors:
        t[:, ids] = 0
    side = torch.cuda.Stream()
    q = wdev.fill_q(wl, 0)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        K.kv_q4_scatter(sh, img, *s.tensors, s.P, ids)
    for _ in range(20):
        K.paged_decode_attn(sh, s.plan, q, s.pool.k, s.pool.v, s.out, s.ws, layer=0, k_params=s.pool.kp,
                            v_params=s.pool.vp)
    torch.cuda.current_stream().wait_stream(side)
    K.paged_decode_attn(sh, s.plan, q, s.pool.k, s.pool.v, s.out, s.ws, layer=0, k_params=s.pool.kp,
                        v_params=s.pool.vp)
    torch.cuda.synchronize()
    for got, w in zip(s.host(), want):
        assert np.array_equal(got.view(np.uint8), w.view(np.uint8))
    assert torch.equal(s.out, ref)
