"""Shared set-up for the GPU tests: build the library's tables and plan, fill the
pool and the queries on the device, run paged_decode_attn through the C ABI."""
import sys

import numpy as np

from shared_paged_kv_amd import _lib as K
from workload import device as wdev


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Case:
    def __init__(self, wl, layers=None):
        import torch
        self.wl = wl
        self.T = K.build_tables(wl.shape, wl.agents)
        a = self.T.arrays
        self.plan = K.DevicePlan(self.T)
        self.pool = wdev.Pool(wl, a["phys_agent"], a["phys_block"], a["phys_ntok"], a["n_dedup"], layers=layers)
        self.ws = torch.empty(max(1, K.workspace_bytes(wl.shape, self.plan)), dtype=torch.uint8, device="cuda")
        self.out = torch.empty((wl.n_agents, wl.shape.n_q_heads, wl.shape.head_dim), dtype=torch.float32,
                               device="cuda")
        self.qseeds = None

    def q(self, layer):
        import torch
        if self.qseeds is None:
            self.qseeds = torch.from_numpy(wdev.query_seeds(self.wl).view(np.int32)).cuda()
        return wdev.fill_q(self.wl, layer, seeds=self.qseeds)

    def run(self, layer=0, q=None):
        import torch
        q = self.q(layer) if q is None else q
        K.paged_decode_attn(self.wl.shape, self.plan, q, self.pool.k, self.pool.v, self.out, self.ws, layer=layer,
                            k_params=self.pool.kp, v_params=self.pool.vp)
        torch.cuda.synchronize()
        return self.out.cpu().numpy().astype(np.float64)
