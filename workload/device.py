"""Device-resident synthetic inputs: the filler in ``libkvgen.so`` writes, on the
GPU, exactly the values ``workload.spec`` / ``workload.rng`` give on the host.

Pools are laid out as the decode library reads them ([layer][phys][kv_head]
[block][head_dim], bf16 or Q4 codes + fp16 (scale, zero) params).  Which
content a physical block holds is read off the table that assigned it
(first-occurrence agent and logical block, or the delta's owner): the seed of
that logical block.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import rng as _rng
from . import spec as _spec

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvgen.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m shared_paged_kv_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i = C.c_void_p, C.c_int
        L.kvgen_fill_bf16.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, vp]
        L.kvgen_fill_q4.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
        L.kvgen_fill_q.argtypes = [vp, vp, i, i, i, i, vp]
        L.kvgen_read_probe.argtypes = [vp, C.c_int64, vp, i, i, i, vp]
        for f in (L.kvgen_fill_bf16, L.kvgen_fill_q4, L.kvgen_fill_q, L.kvgen_read_probe):
            f.restype = C.c_int
        _lib = L
    return _lib


def _stream():
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def phys_seeds(wl, phys_agent, phys_block, n_dedup) -> np.ndarray:
    """[n_phys, 4] uint32 content seeds of the physical blocks."""
    n = len(phys_agent)
    out = np.empty((n, 4), np.uint32)
    for p in range(n):
        j, b = int(phys_agent[p]), int(phys_block[p])
        s = wl.blk_delta_seed[j][b] if p >= n_dedup else wl.blk_seed[j][b]
        out[p] = np.frombuffer(s, dtype="<u4")
    return out


class Pool:
    """K and V pools of a workload on the GPU (all layers allocated)."""

    def __init__(self, wl, phys_agent, phys_block, phys_ntok, n_dedup, device="cuda", layers=None, capacity=None):
        """capacity: physical blocks allocated (default n_phys); blocks past
        n_phys are left unfilled, for blocks created after the build."""
        import torch
        sh = wl.shape
        self.wl, self.n_phys = wl, len(phys_agent)
        P, H, B, D, Lyr = self.n_phys, sh.n_kv_heads, sh.block_tokens, sh.head_dim, sh.n_layers
        self.seeds = torch.from_numpy(phys_seeds(wl, phys_agent, phys_block, n_dedup).view(np.int32)).to(device)
        self.ntok = torch.from_numpy(np.ascontiguousarray(phys_ntok, np.int32)).to(device)
        Pa = max(P, 1, capacity or 0)
        self.capacity = Pa
        if sh.kv_dtype == _spec.BF16:
            self.k = torch.empty((Lyr, Pa, H, B, D), dtype=torch.bfloat16, device=device)
            self.v = torch.empty_like(self.k)
            self.kp = self.vp = None
        else:
            self.k = torch.empty((Lyr, Pa, H, B, D // 2), dtype=torch.uint8, device=device)
            self.v = torch.empty_like(self.k)
            self.kp = torch.empty((Lyr, Pa, H, B, D // 64, 2), dtype=torch.float16, device=device)
            self.vp = torch.empty_like(self.kp)
        for layer in (range(Lyr) if layers is None else layers):
            self.fill_layer(layer)

    def fill_layer(self, layer):
        sh = self.wl.shape
        L = lib()
        args = (self.seeds.data_ptr(), self.ntok.data_ptr(), self.n_phys, self.capacity, int(layer), sh.n_kv_heads,
                sh.block_tokens, sh.head_dim)
        for sel, t, tp in ((_rng.SEL_K, self.k, self.kp), (_rng.SEL_V, self.v, self.vp)):
            if sh.kv_dtype == _spec.BF16:
                rc = L.kvgen_fill_bf16(t.data_ptr(), *args, sel, _stream())
            else:
                rc = L.kvgen_fill_q4(t.data_ptr(), tp.data_ptr(), *args, sel, _stream())
            if rc:
                raise RuntimeError(f"kvgen fill failed ({rc})")

    @property
    def nbytes(self):
        n = self.k.numel() * self.k.element_size() * 2
        if self.kp is not None:
            n += self.kp.numel() * self.kp.element_size() * 2
        return n


def query_seeds(wl) -> np.ndarray:
    out = np.empty((wl.n_agents, 4), np.uint32)
    import struct
    for j in range(wl.n_agents):
        s = _spec._h(b"query", wl.name.encode(), struct.pack("<qi", wl.seed, j))
        out[j] = np.frombuffer(s, dtype="<u4")
    return out


def fill_q(wl, layer, out=None, seeds=None, device="cuda"):
    """Decode queries of one layer on the GPU: bf16 [n, Hq, d] (== spec.q_bits)."""
    import torch
    sh = wl.shape
    if out is None:
        out = torch.empty((wl.n_agents, sh.n_q_heads, sh.head_dim), dtype=torch.bfloat16, device=device)
    if seeds is None:
        seeds = torch.from_numpy(query_seeds(wl).view(np.int32)).to(device)
    rc = lib().kvgen_fill_q(out.data_ptr(), seeds.data_ptr(), wl.n_agents, int(layer), sh.n_q_heads, sh.head_dim,
                            _stream())
    if rc:
        raise RuntimeError(f"kvgen q fill failed ({rc})")
    return out


def read_probe(buf, out, grid: int, nontemporal: bool, chunked: bool = False) -> None:
    """One launch of the plain read probe over all of ``buf`` (a CUDA uint8
    tensor, size a multiple of 16) on the current stream; ``out``: a CUDA tensor
    of at least 4 bytes.  chunked: each workgroup reads a contiguous share
    (non-temporal) instead of the grid-stride sweep."""
    if not (buf.is_cuda and out.is_cuda and buf.is_contiguous()) or out.numel() * out.element_size() < 4:
        raise ValueError("read_probe: buf must be a contiguous CUDA tensor and out at least 4 device bytes")
    nbytes = buf.numel() * buf.element_size()
    rc = lib().kvgen_read_probe(C.c_void_p(buf.data_ptr()), nbytes, C.c_void_p(out.data_ptr()), grid,
                                1 if nontemporal else 0, 1 if chunked else 0, _stream())
    if rc:
        raise RuntimeError(f"kvgen_read_probe failed ({rc})")
