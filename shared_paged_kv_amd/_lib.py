"""ctypes binding of libkvpool.so (include/kvpool.h, kvpool_lifecycle.h, kvpool_mirror.h).

Argument marshalling only: numpy arrays and torch tensors are turned into the
pointers, sizes and stream the C ABI takes.  Every step of the decode path runs
in the library's kernels.  Loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVPOOL_LIB names another build of the library to load instead (for example the
# host-only sanitizer build of the control plane, which has no device entry points)
LIB_PATH = os.environ.get("KVPOOL_LIB") or os.path.join(_HERE, "libkvpool.so")

KVP_OK, KVP_EINVAL, KVP_ETIER, KVP_ENOMEM, KVP_EWORKSPACE, KVP_EHIP, KVP_EFULL, KVP_EIO = 0, -1, -2, -3, -4, -5, -6, -7
KVP_BF16, KVP_Q4G64, KVP_F32 = 0, 1, 2
KVP_GLOBAL, KVP_GROUP, KVP_PRIVATE = 0, 1, 2
KVP_PREFIX, KVP_SEGMENT = 0, 1

P32 = C.POINTER(C.c_int32)


class kvp_shape(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("block_tokens", C.c_int32), ("kv_dtype", C.c_int32),
                ("rope_theta", C.c_float)]


class kvp_span(C.Structure):
    _fields_ = [("tier", C.c_int32), ("group", C.c_int32), ("kind", C.c_int32), ("n_tokens", C.c_int32),
                ("tokens", P32)]


class kvp_agent(C.Structure):
    _fields_ = [("n_spans", C.c_int32), ("spans", C.POINTER(kvp_span)), ("n_delta", C.c_int32),
                ("delta_blocks", P32)]


class kvp_item(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("blk_begin", "blk_end", "cons_begin", "cons_end", "part_base", "mask_base", "mask_stride", "rows")]


class kvp_tables_view(C.Structure):
    _fields_ = [("n_agents", C.c_int32), ("max_blocks", C.c_int32), ("n_phys", C.c_int32),
                ("n_dedup", C.c_int32), ("n_delta", C.c_int32),
                ("n_blocks", P32), ("block_table", P32), ("delta_table", P32), ("ntok", P32),
                ("dst_pos0", P32), ("shift", P32), ("src_pos0", P32), ("refcount", P32),
                ("phys_ntok", P32), ("phys_agent", P32), ("phys_block", P32),
                ("n_items", C.c_int32), ("n_plan_blocks", C.c_int32), ("n_cons", C.c_int32),
                ("n_qcons", C.c_int32), ("n_mask_words", C.c_int32), ("n_part_rows", C.c_int32),
                ("n_comb", C.c_int32),
                ("items", C.POINTER(kvp_item)), ("plan_blocks", P32), ("cons", P32), ("qcons", P32),
                ("mask", C.POINTER(C.c_uint32)), ("comb_ptr", P32), ("comb_rows", P32),
                ("n_qcons_shifted", C.c_int32), ("class_items", C.c_int32 * 6), ("unit_span", C.c_int32),
                ("unique_kv_bytes", C.c_int64), ("plan_ntok", P32), ("cons_row", P32),
                ("rope_cs", C.POINTER(C.c_float)), ("n_rope_cs", C.c_int32)]


class kvp_plan_dev(C.Structure):
    _fields_ = [("n_agents", C.c_int32), ("n_phys", C.c_int32), ("n_items", C.c_int32),
                ("n_qcons", C.c_int32), ("n_qcons_shifted", C.c_int32), ("n_part_rows", C.c_int32),
                ("class_items", C.c_int32 * 6), ("unit_span", C.c_int32),
                ("items", C.c_void_p), ("plan_blocks", C.c_void_p), ("cons", C.c_void_p),
                ("qcons", C.c_void_p), ("mask", C.c_void_p), ("phys_ntok", C.c_void_p),
                ("comb_ptr", C.c_void_p), ("comb_rows", C.c_void_p), ("plan_ntok", C.c_void_p),
                ("cons_row", C.c_void_p), ("rope_cs", C.c_void_p),
                ("n_plan_blocks", C.c_int32), ("n_cons", C.c_int32), ("n_mask_words", C.c_int32),
                ("n_comb", C.c_int32)]


# the device arrays of a kvp_plan_dev
PLAN_ARRAYS = ("items", "plan_blocks", "cons", "qcons", "mask", "phys_ntok", "comb_ptr", "comb_rows", "plan_ntok",
               "cons_row", "rope_cs")


class kvp_append_ops(C.Structure):
    _fields_ = [("n_copies", C.c_int32), ("copies", P32), ("n_writes", C.c_int32), ("writes", P32)]


class kvp_audit(C.Structure):
    _fields_ = [("n_allocated", C.c_int32), ("n_leaked", C.c_int32), ("n_mismatched", C.c_int32),
                ("n_live_agents", C.c_int32), ("leaked_tokens", C.c_int64)]


EXPORTS = ["kvpool_build_tables", "kvpool_tables_view", "kvpool_tables_free", "kv_rerotate",
           "paged_decode_attn_workspace_bytes", "paged_decode_attn", "paged_decode_attn_phases",
           "paged_decode_attn_noalloc", "kvpool_last_error",
           "kvpool_fnv1a64_words", "kvpool_debug_set_hash_bits", "kvpool_device_checks_enabled",
           "kvpool_debug_take_device_errors",
           # include/kvpool_lifecycle.h
           "kvpool_pool_create", "kvpool_pool_free", "kvpool_append", "kvpool_destroy", "kvpool_lose",
           "kvpool_audit", "kvpool_reclaim", "kvpool_pool_tables", "kv_append",
           # include/kvpool_mirror.h
           "kv_diff_blocks", "kv_restore", "kvpool_restore_list",
           # include/kvpool_persist.h
           "kvpool_q4_image_bytes", "kv_q4_gather", "kv_q4_scatter", "kvpool_q4_save_file", "kvpool_q4_load_file"]

_lib = None


class KvpError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"kvpool error {code}: {msg}")
        self.code = code


class _HostOnly:
    """Binding target for a build of the host control plane alone: declarations
    of the device entry points it does not export land on a throwaway object
    (calling one through the library raises AttributeError)."""

    def __init__(self, L):
        object.__setattr__(self, "_L", L)

    def __getattr__(self, name):
        try:
            return getattr(self._L, name)
        except AttributeError:
            return _Absent()


class _Absent:
    pass


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m shared_paged_kv_amd.build`")
        L = C.CDLL(LIB_PATH)
        # a host-only build (no device entry points) binds what it exports
        B = L if hasattr(L, "paged_decode_attn") else _HostOnly(L)
        B.kvpool_build_tables.argtypes = [C.POINTER(kvp_shape), C.POINTER(kvp_agent), C.c_int32, C.POINTER(C.c_void_p)]
        B.kvpool_build_tables.restype = C.c_int
        B.kvpool_tables_view.argtypes = [C.c_void_p, C.POINTER(kvp_tables_view)]
        B.kvpool_tables_view.restype = C.c_int
        B.kvpool_tables_free.argtypes = [C.c_void_p]
        B.kvpool_tables_free.restype = None
        B.kv_rerotate.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_float,
                                  C.c_int32, C.c_int32, C.c_void_p]
        B.kv_rerotate.restype = C.c_int
        B.paged_decode_attn_workspace_bytes.argtypes = [C.POINTER(kvp_shape), C.POINTER(kvp_plan_dev),
                                                        C.POINTER(C.c_size_t)]
        B.paged_decode_attn_workspace_bytes.restype = C.c_int
        B.paged_decode_attn.argtypes = [C.POINTER(kvp_shape), C.POINTER(kvp_plan_dev), C.c_void_p, C.c_void_p,
                                        C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_float, C.c_void_p,
                                        C.c_void_p, C.c_size_t, C.c_void_p]
        B.paged_decode_attn.restype = C.c_int
        B.paged_decode_attn_phases.argtypes = [C.POINTER(kvp_shape), C.POINTER(kvp_plan_dev), C.c_void_p, C.c_void_p,
                                               C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_float, C.c_void_p,
                                               C.c_void_p, C.c_size_t, C.c_uint32, C.c_void_p]
        B.paged_decode_attn_phases.restype = C.c_int
        B.paged_decode_attn_noalloc.argtypes = [C.POINTER(kvp_shape), C.POINTER(kvp_plan_dev), C.c_void_p,
                                                C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                                C.c_float, C.c_void_p, C.c_void_p]
        B.paged_decode_attn_noalloc.restype = C.c_int
        B.kvpool_last_error.argtypes = []
        B.kvpool_last_error.restype = C.c_char_p
        B.kvpool_fnv1a64_words.argtypes = [C.POINTER(C.c_uint32), C.c_int64]
        B.kvpool_fnv1a64_words.restype = C.c_uint64
        B.kvpool_debug_set_hash_bits.argtypes = [C.c_int32]
        B.kvpool_debug_set_hash_bits.restype = C.c_int
        B.kvpool_device_checks_enabled.argtypes = []
        B.kvpool_device_checks_enabled.restype = C.c_int
        B.kvpool_debug_take_device_errors.argtypes = [C.c_void_p, C.c_void_p]
        B.kvpool_debug_take_device_errors.restype = C.c_int
        B.kvpool_pool_create.argtypes = [C.c_void_p, C.POINTER(kvp_shape), C.c_int32, C.POINTER(C.c_void_p)]
        B.kvpool_pool_create.restype = C.c_int
        B.kvpool_pool_free.argtypes = [C.c_void_p]
        B.kvpool_pool_free.restype = None
        B.kvpool_append.argtypes = [C.c_void_p, C.c_int32, P32, C.POINTER(kvp_append_ops)]
        B.kvpool_append.restype = C.c_int
        B.kvpool_destroy.argtypes = [C.c_void_p, C.c_int32]
        B.kvpool_destroy.restype = C.c_int
        B.kvpool_lose.argtypes = [C.c_void_p, C.c_int32]
        B.kvpool_lose.restype = C.c_int
        B.kvpool_audit.argtypes = [C.c_void_p, C.POINTER(kvp_audit), P32, C.c_int32]
        B.kvpool_audit.restype = C.c_int
        B.kvpool_reclaim.argtypes = [C.c_void_p]
        B.kvpool_reclaim.restype = C.c_int
        B.kvpool_pool_tables.argtypes = [C.c_void_p, C.POINTER(C.c_void_p)]
        B.kvpool_pool_tables.restype = C.c_int
        B.kv_append.argtypes = [C.POINTER(kvp_shape), C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32,
                                C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p]
        B.kv_append.restype = C.c_int
        B.kv_diff_blocks.argtypes = [C.POINTER(kvp_shape), C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                     C.c_int32, C.c_void_p, C.c_int32, C.c_float, C.c_void_p, C.c_void_p]
        B.kv_diff_blocks.restype = C.c_int
        B.kv_restore.argtypes = [C.POINTER(kvp_shape), C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32,
                                 C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p]
        B.kv_restore.restype = C.c_int
        B.kvpool_restore_list.argtypes = [C.c_void_p, P32, C.c_int32, P32, C.c_int32]
        B.kvpool_restore_list.restype = C.c_int
        B.kvpool_q4_image_bytes.argtypes = [C.POINTER(kvp_shape), C.c_int32]
        B.kvpool_q4_image_bytes.restype = C.c_int64
        B.kv_q4_gather.argtypes = [C.POINTER(kvp_shape), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                   P32, C.c_int32, C.c_void_p, C.c_void_p]
        B.kv_q4_gather.restype = C.c_int
        B.kv_q4_scatter.argtypes = [C.POINTER(kvp_shape), C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_int32, P32, C.c_void_p]
        B.kv_q4_scatter.restype = C.c_int
        B.kvpool_q4_save_file.argtypes = [C.POINTER(kvp_shape), C.c_char_p, C.c_char_p, C.c_void_p, P32, C.c_int32]
        B.kvpool_q4_save_file.restype = C.c_int
        B.kvpool_q4_load_file.argtypes = [C.POINTER(kvp_shape), C.c_char_p, C.c_char_p, C.c_void_p, C.c_int64, P32,
                                          C.c_int32]
        B.kvpool_q4_load_file.restype = C.c_int
        _lib = L
    return _lib


def _check(rc):
    if rc != KVP_OK:
        raise KvpError(rc, lib().kvpool_last_error().decode())


def make_shape(s) -> kvp_shape:
    return kvp_shape(s.n_layers, s.n_q_heads, s.n_kv_heads, s.head_dim, s.block_tokens, s.kv_dtype,
                     float(s.rope_theta))


# ---------------------------------------------------------------------------
# tables


class Tables:
    """Owns a kvp_tables handle; ``arrays`` holds numpy copies of every view array."""

    def __init__(self, handle, view: kvp_tables_view):
        self._h = handle
        v = view
        n, M, P = v.n_agents, v.max_blocks, v.n_phys

        def arr(ptr, count, dt=np.int32):
            if count == 0:
                return np.zeros(0, dt)
            return np.ctypeslib.as_array(ptr, shape=(count,)).astype(dt, copy=True)

        self.n_agents, self.max_blocks, self.n_phys = n, M, P
        self.n_dedup, self.n_delta = v.n_dedup, v.n_delta
        a = dict(n_agents=n, max_blocks=M, n_phys=P, n_dedup=v.n_dedup, n_delta=v.n_delta)
        a["n_blocks"] = arr(v.n_blocks, n)
        for k in ("block_table", "delta_table", "ntok", "dst_pos0", "shift"):
            a[k] = arr(getattr(v, k), n * M).reshape(n, M)
        for k in ("src_pos0", "refcount", "phys_ntok", "phys_agent", "phys_block"):
            a[k] = arr(getattr(v, k), P)
        items = np.zeros((v.n_items, 8), np.int32)
        if v.n_items:
            raw = C.cast(v.items, P32)
            items = np.ctypeslib.as_array(raw, shape=(v.n_items * 8,)).reshape(v.n_items, 8).copy()
        a["items"] = items
        a["plan_blocks"] = arr(v.plan_blocks, v.n_plan_blocks)
        a["cons"] = arr(v.cons, v.n_cons)
        a["qcons"] = arr(v.qcons, 2 * v.n_qcons)
        a["mask"] = arr(v.mask, v.n_mask_words, np.uint32)
        a["comb_ptr"] = arr(v.comb_ptr, n + 1)
        a["comb_rows"] = arr(v.comb_rows, v.n_comb)
        a["plan_ntok"] = arr(v.plan_ntok, v.n_plan_blocks)
        a["cons_row"] = arr(v.cons_row, v.n_cons)
        a["rope_cs"] = arr(v.rope_cs, v.n_rope_cs, np.float32)
        a["class_items"] = np.array(list(v.class_items), np.int32)
        a["n_part_rows"] = v.n_part_rows
        a["n_qcons"] = v.n_qcons
        a["n_qcons_shifted"] = v.n_qcons_shifted
        a["unit_span"] = v.unit_span
        a["unique_kv_bytes"] = int(v.unique_kv_bytes)
        self.arrays = a

    def __getitem__(self, k):
        return self.arrays[k]

    def close(self):
        if self._h:
            lib().kvpool_tables_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def build_tables(shape, agents) -> Tables:
    """shape: object with the kvp_shape fields; agents: objects with ``spans``
    (tier, group, kind, tokens) and ``delta_blocks``."""
    L = lib()
    keep = []
    c_agents = (kvp_agent * max(1, len(agents)))()
    for j, ag in enumerate(agents):
        spans = (kvp_span * max(1, len(ag.spans)))()
        for i, sp in enumerate(ag.spans):
            t = np.ascontiguousarray(sp.tokens, dtype=np.int32)
            keep.append(t)
            spans[i] = kvp_span(int(sp.tier), int(sp.group), int(sp.kind), len(t), t.ctypes.data_as(P32))
        d = np.ascontiguousarray(ag.delta_blocks, dtype=np.int32)
        keep += [spans, d]
        c_agents[j] = kvp_agent(len(ag.spans), spans, len(d), d.ctypes.data_as(P32))
    sh = make_shape(shape)
    h = C.c_void_p()
    _check(L.kvpool_build_tables(C.byref(sh), c_agents, len(agents), C.byref(h)))
    v = kvp_tables_view()
    rc = L.kvpool_tables_view(h, C.byref(v))
    if rc:
        L.kvpool_tables_free(h)
        _check(rc)
    return Tables(h, v)


def _tables_from_handle(h) -> Tables:
    L = lib()
    v = kvp_tables_view()
    rc = L.kvpool_tables_view(h, C.byref(v))
    if rc:
        L.kvpool_tables_free(h)
        _check(rc)
    return Tables(h, v)


class BlockPool:
    """Owns a kvp_pool handle: the block lifecycle (append with copy-on-write,
    destroy, lose, audit, reclaim) over tables built by build_tables."""

    def __init__(self, tables: Tables, shape, capacity: int):
        self.shape = shape
        self.capacity = int(capacity)
        sh = make_shape(shape)
        h = C.c_void_p()
        _check(lib().kvpool_pool_create(tables._h, C.byref(sh), self.capacity, C.byref(h)))
        self._h = h

    def append(self, agents):
        """One token for each listed agent (row i = agents[i]).  Returns
        (copies [n, 2], writes [n, 4]) as numpy int32 copies."""
        a = np.ascontiguousarray(agents, dtype=np.int32)
        ops = kvp_append_ops()
        _check(lib().kvpool_append(self._h, len(a), a.ctypes.data_as(P32), C.byref(ops)))
        cp = np.ctypeslib.as_array(ops.copies, shape=(2 * ops.n_copies,)).copy() if ops.n_copies else np.zeros(0, np.int32)
        wr = np.ctypeslib.as_array(ops.writes, shape=(4 * ops.n_writes,)).copy() if ops.n_writes else np.zeros(0, np.int32)
        return cp.reshape(-1, 2), wr.reshape(-1, 4)

    def destroy(self, agent: int):
        _check(lib().kvpool_destroy(self._h, int(agent)))

    def lose(self, agent: int):
        _check(lib().kvpool_lose(self._h, int(agent)))

    def audit(self, max_ids: int = 0):
        au = kvp_audit()
        ids = np.zeros(max(1, max_ids), np.int32)
        _check(lib().kvpool_audit(self._h, C.byref(au), ids.ctypes.data_as(P32) if max_ids else None, int(max_ids)))
        out = dict(n_allocated=au.n_allocated, n_leaked=au.n_leaked, n_mismatched=au.n_mismatched,
                   n_live_agents=au.n_live_agents, leaked_tokens=int(au.leaked_tokens))
        if max_ids:
            out["leaked_ids"] = ids[:min(max_ids, au.n_leaked)].copy()
        return out

    def reclaim(self) -> int:
        rc = lib().kvpool_reclaim(self._h)
        if rc < 0:
            _check(rc)
        return int(rc)

    def tables(self) -> Tables:
        h = C.c_void_p()
        _check(lib().kvpool_pool_tables(self._h, C.byref(h)))
        return _tables_from_handle(h)

    def close(self):
        if self._h:
            lib().kvpool_pool_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fnv1a64_words(words) -> int:
    w = np.ascontiguousarray(words, dtype=np.uint32)
    return int(lib().kvpool_fnv1a64_words(w.ctypes.data_as(C.POINTER(C.c_uint32)), len(w)))


def set_hash_bits(bits: int):
    _check(lib().kvpool_debug_set_hash_bits(int(bits)))


def device_checks_enabled() -> bool:
    """True when the loaded library is the checked build (kernel bounds checks)."""
    return bool(lib().kvpool_device_checks_enabled())


def take_device_errors() -> int:
    """The current device's error word of the checked build (bits 1: item ranges,
    2: block ids or token counts, 4: consumers, 8: combine lists), cleared;
    synchronises the current stream.  Always 0 from the ordinary build."""
    import torch
    dst = torch.zeros(1, dtype=torch.int32, device="cuda")
    _check(lib().kvpool_debug_take_device_errors(C.c_void_p(dst.data_ptr()), _stream()))
    return int(dst.item()) & 0xffffffff


# ---------------------------------------------------------------------------
# device side (torch tensors for memory and streams)


def _stream():
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, name="device argument"):
    """Device pointer of a contiguous tensor on the GPU (None -> NULL).  The
    library cannot see the extent of a device buffer, so anything else is
    refused here rather than handed to a kernel."""
    if t is None:
        return C.c_void_p(0)
    if not t.is_contiguous():
        raise KvpError(KVP_EINVAL, f"{name}: must be contiguous")
    if not getattr(t, "is_cuda", False):
        raise KvpError(KVP_EINVAL, f"{name}: expected a tensor in device memory")
    return C.c_void_p(t.data_ptr())


def _dev(specs):
    """Checked pointers of (tensor, name, dtypes, numel) tuples: every tensor
    (None allowed when numel is 0) must have one of dtypes and at least numel
    elements, the extent the call reads or writes per the layouts in kvpool.h;
    then each goes through _ptr."""
    for t, name, dtypes, numel in specs:
        if t is None:
            if numel > 0:
                raise KvpError(KVP_EINVAL, f"{name}: required")
            continue
        if t.dtype not in dtypes:
            raise KvpError(KVP_EINVAL, f"{name}: dtype {t.dtype}, expected one of {list(dtypes)}")
        if t.numel() < numel:
            raise KvpError(KVP_EINVAL, f"{name}: {t.numel()} elements, the call uses {numel}")
    return [_ptr(t, name) for t, name, _, _ in specs]


class DevicePlan:
    """Device copies of a Tables' work plan plus the kvp_plan_dev pointing at them."""

    def __init__(self, tables: Tables, device="cuda"):
        import torch
        a = tables.arrays
        self.tensors = {}

        def up(name, x, dtype=torch.int32):
            x = np.ascontiguousarray(x)
            if x.size == 0:
                x = np.zeros(1, x.dtype)
            t = torch.from_numpy(x.view(np.int32) if x.dtype == np.uint32 else x).to(device)
            self.tensors[name] = t
            return t

        up("items", a["items"].reshape(-1))
        up("plan_blocks", a["plan_blocks"])
        up("cons", a["cons"])
        up("qcons", a["qcons"])
        up("mask", a["mask"])
        up("phys_ntok", a["phys_ntok"])
        up("comb_ptr", a["comb_ptr"])
        up("comb_rows", a["comb_rows"])
        up("plan_ntok", a["plan_ntok"])
        up("cons_row", a["cons_row"])
        up("rope_cs", a["rope_cs"])
        s = kvp_plan_dev()
        s.n_agents = a["n_agents"]
        s.n_phys = a["n_phys"]
        s.n_items = int(a["items"].shape[0])
        s.n_qcons = int(a["n_qcons"])
        s.n_qcons_shifted = int(a["n_qcons_shifted"])
        s.unit_span = int(a["unit_span"])
        s.n_part_rows = int(a["n_part_rows"])
        s.n_plan_blocks = int(a["plan_blocks"].shape[0])
        s.n_cons = int(a["cons"].shape[0])
        s.n_mask_words = int(a["mask"].shape[0])
        s.n_comb = int(a["comb_rows"].shape[0])
        for i in range(6):
            s.class_items[i] = int(a["class_items"][i])
        for k in PLAN_ARRAYS:
            setattr(s, k, self.tensors[k].data_ptr())
        self.c = s


def _bf16():
    """dtypes accepted for a bf16 argument: bf16 or its 16-bit integer view."""
    import torch
    return (torch.bfloat16, torch.int16)


def _slots(shape, blocks):
    """Token slots of a [n_layers][blocks][Hkv][B] pool (0 for negative blocks:
    the library refuses those itself)."""
    return shape.n_layers * max(0, int(blocks)) * shape.n_kv_heads * shape.block_tokens


def _q4_args(shape, pool_blocks, n, image, k_codes, v_codes, k_params, v_params):
    """Checked device pointers of the Q4 pool tensors, after checking that the
    host image holds n blocks."""
    import torch
    if n > 0:
        need = q4_image_bytes(shape, n)
        have = 0 if image is None else (image.nbytes if isinstance(image, np.ndarray)
                                        else image.numel() * image.element_size())
        if have < need:
            raise KvpError(KVP_EINVAL, f"image: {have} bytes, {n} blocks need {need}")
    slots = _slots(shape, pool_blocks) if n > 0 else 0
    codes_n, par_n = slots * shape.head_dim // 2, slots * (shape.head_dim // 64) * 2
    return _dev([(k_codes, "k_codes", (torch.uint8,), codes_n), (v_codes, "v_codes", (torch.uint8,), codes_n),
                 (k_params, "k_params", (torch.float16,), par_n), (v_params, "v_params", (torch.float16,), par_n)])


def kv_append(shape, k_pool, v_pool, capacity, copies, writes, k_new, v_new, n_rows):
    """Device work of one BlockPool.append: copies / writes are device int32
    tensors (or None when empty), k_new / v_new device bf16 [L, n_rows, Hkv, d]."""
    import torch
    sh = make_shape(shape)
    nc = 0 if copies is None else copies.numel() // 2
    nw = 0 if writes is None else writes.numel() // 4
    pool_n = _slots(shape, capacity) * shape.head_dim
    new_n = shape.n_layers * max(0, int(n_rows)) * shape.n_kv_heads * shape.head_dim if nw else 0
    bf, i32 = _bf16(), (torch.int32,)
    pk, pv, pc, pw, nk, nv = _dev([(k_pool, "k_pool", bf, pool_n), (v_pool, "v_pool", bf, pool_n),
                                   (copies, "copies", i32, 2 * nc), (writes, "writes", i32, 4 * nw),
                                   (k_new, "k_new", bf, new_n), (v_new, "v_new", bf, new_n)])
    _check(lib().kv_append(C.byref(sh), pk, pv, int(capacity), pc, nc, pw, nw, nk, nv, int(n_rows), _stream()))


def restore_list(tables: Tables, agents) -> np.ndarray:
    """[n, 4] int32 restore entries (source physical id, shift, valid tokens,
    destination block) of the listed agents (an int: one agent), ordered by
    source; destinations number the agents' logical blocks in list order."""
    L = lib()
    ag = np.ascontiguousarray(np.atleast_1d(np.asarray(agents, np.int32)))
    pa = ag.ctypes.data_as(P32)
    n = L.kvpool_restore_list(tables._h, pa, len(ag), None, 0)
    if n < 0:
        _check(n)
    out = np.zeros(max(1, 4 * n), np.int32)
    _check(min(0, L.kvpool_restore_list(tables._h, pa, len(ag), out.ctypes.data_as(P32), n)))
    return out[:4 * n].reshape(n, 4)


def kv_restore(shape, k_pool, v_pool, pool_blocks, entries, dst_k, dst_v, dst_blocks):
    """entries: device int32 [n, 4]; dst_k / dst_v: device bf16 [L, dst_blocks, Hkv, B, d]."""
    import torch
    sh = make_shape(shape)
    n = 0 if entries is None else entries.numel() // 4
    bf = _bf16()
    src_n = _slots(shape, pool_blocks) * shape.head_dim if n else 0
    dst_n = _slots(shape, dst_blocks) * shape.head_dim if n else 0
    pk, pv, pe, dk, dv = _dev([(k_pool, "k_pool", bf, src_n), (v_pool, "v_pool", bf, src_n),
                               (entries, "entries", (torch.int32,), 4 * n), (dst_k, "dst_k", bf, dst_n),
                               (dst_v, "dst_v", bf, dst_n)])
    _check(lib().kv_restore(C.byref(sh), pk, pv, int(pool_blocks), pe, n, dk, dv, int(dst_blocks), _stream()))


def kv_diff_blocks(shape, k_pool, v_pool, pool_blocks, cand_k, cand_v, cand_blocks, pairs, tau, flags):
    """pairs: device int32 [n, 3]; flags: device int32 [n]."""
    import torch
    sh = make_shape(shape)
    n = 0 if pairs is None else pairs.numel() // 3
    bf, i32 = _bf16(), (torch.int32,)
    src_n = _slots(shape, pool_blocks) * shape.head_dim if n else 0
    cand_n = _slots(shape, cand_blocks) * shape.head_dim if n else 0
    pk, pv, ck, cv, pp, pf = _dev([(k_pool, "k_pool", bf, src_n), (v_pool, "v_pool", bf, src_n),
                                   (cand_k, "cand_k", bf, cand_n), (cand_v, "cand_v", bf, cand_n),
                                   (pairs, "pairs", i32, 3 * n), (flags, "flags", i32, n)])
    _check(lib().kv_diff_blocks(C.byref(sh), pk, pv, int(pool_blocks), ck, cv, int(cand_blocks), pp, n, float(tau), pf,
                                _stream()))


def _hptr(x):
    """Host pointer of a CPU torch tensor or a numpy array (None -> NULL)."""
    if x is None:
        return C.c_void_p(0)
    if isinstance(x, np.ndarray):
        return C.c_void_p(x.ctypes.data)
    return C.c_void_p(x.data_ptr())


def q4_image_bytes(shape, n: int) -> int:
    sh = make_shape(shape)
    r = lib().kvpool_q4_image_bytes(C.byref(sh), int(n))
    _check(min(0, r))
    return int(r)


def kv_q4_gather(shape, k_codes, v_codes, k_params, v_params, pool_blocks, ids, image):
    """Q4 pool blocks ids (host ints) -> image (host uint8, pinned for an
    asynchronous copy), enqueued on the current stream."""
    sh = make_shape(shape)
    ids = np.ascontiguousarray(ids, np.int32)
    ptrs = _q4_args(shape, pool_blocks, len(ids), image, k_codes, v_codes, k_params, v_params)
    _check(lib().kv_q4_gather(C.byref(sh), *ptrs, int(pool_blocks), ids.ctypes.data_as(P32), len(ids), _hptr(image),
                              _stream()))


def kv_q4_scatter(shape, image, k_codes, v_codes, k_params, v_params, pool_blocks, ids):
    """image (host) -> Q4 pool blocks ids, enqueued on the current stream."""
    sh = make_shape(shape)
    ids = np.ascontiguousarray(ids, np.int32)
    ptrs = _q4_args(shape, pool_blocks, len(ids), image, k_codes, v_codes, k_params, v_params)
    _check(lib().kv_q4_scatter(C.byref(sh), _hptr(image), len(ids), *ptrs, int(pool_blocks),
                               ids.ctypes.data_as(P32), _stream()))


def q4_save_file(shape, path, agent, image, ntok):
    sh = make_shape(shape)
    nt = np.ascontiguousarray(ntok, np.int32)
    _check(lib().kvpool_q4_save_file(C.byref(sh), os.fsencode(path), agent.encode(), _hptr(image),
                                     nt.ctypes.data_as(P32), len(nt)))


def q4_load_file(shape, path, agent=None, image=None):
    """Returns the file's block count n; with image (host, large enough) also
    reads the tensors into it and returns (n, ntok)."""
    sh = make_shape(shape)
    L = lib()
    ag = None if agent is None else agent.encode()
    n = L.kvpool_q4_load_file(C.byref(sh), os.fsencode(path), ag, None, 0, None, 0)
    _check(min(0, n))
    if image is None:
        return n
    nt = np.zeros(n, np.int32)
    nbytes = image.nbytes if isinstance(image, np.ndarray) else image.numel() * image.element_size()
    r = L.kvpool_q4_load_file(C.byref(sh), os.fsencode(path), ag, _hptr(image), nbytes, nt.ctypes.data_as(P32), n)
    _check(min(0, r))
    if r != n or nbytes < q4_image_bytes(shape, n):
        raise KvpError(KVP_EINVAL, "image too small for the file")
    return n, nt


def workspace_bytes(shape, plan: DevicePlan) -> int:
    n = C.c_size_t()
    sh = make_shape(shape)
    _check(lib().paged_decode_attn_workspace_bytes(C.byref(sh), C.byref(plan.c), C.byref(n)))
    return int(n.value)


def paged_decode_attn(shape, plan: DevicePlan, q, k_pool, v_pool, out, workspace, layer=0, scale=None,
                      k_params=None, v_params=None):
    """q: bf16 [n, Hq, d]; pools per kvpool.h; out float32 [n, Hq, d];
    workspace: a uint8 tensor of at least workspace_bytes()."""
    sh = make_shape(shape)
    if scale is None:
        scale = 1.0 / float(shape.head_dim) ** 0.5
    args = _decode_args(shape, plan, q, k_pool, v_pool, k_params, v_params, out, workspace)
    _check(lib().paged_decode_attn(C.byref(sh), C.byref(plan.c), args[0], args[1], args[2], args[3], args[4],
                                   int(layer), float(scale), args[5], args[6], args[7], _stream()))
    return out


NOALLOC_SCRATCH_BYTES = 128 << 20   # KVP_NOALLOC_SCRATCH_BYTES


def paged_decode_attn_noalloc(shape, plan: DevicePlan, q, k_pool, v_pool, out, layer=0, scale=None,
                              k_params=None, v_params=None):
    """paged_decode_attn on the library's own per-device scratch array (no
    workspace argument, no device allocation).  Calls on one device share that
    array, so calls that overlap on one device race."""
    sh = make_shape(shape)
    if scale is None:
        scale = 1.0 / float(shape.head_dim) ** 0.5
    args = _decode_args(shape, plan, q, k_pool, v_pool, k_params, v_params, out, None)
    _check(lib().paged_decode_attn_noalloc(C.byref(sh), C.byref(plan.c), args[0], args[1], args[2], args[3],
                                           args[4], int(layer), float(scale), args[5], _stream()))
    return out


def _decode_args(shape, plan, q, k_pool, v_pool, k_params, v_params, out, workspace):
    """Checked pointers (q, k_pool, v_pool, k_params, v_params, out, workspace)
    and the workspace size of a decode call."""
    import torch
    c = plan.c
    rows = c.n_agents * shape.n_q_heads * shape.head_dim if c.n_agents > 0 else 0
    slots = shape.n_layers * c.n_phys * shape.n_kv_heads * shape.block_tokens if c.n_items > 0 else 0
    q4 = shape.kv_dtype == KVP_Q4G64
    pool_t, pool_n = ((torch.uint8,), slots * shape.head_dim // 2) if q4 else (_bf16(), slots * shape.head_dim)
    par_n = slots * (shape.head_dim // 64) * 2 if q4 else 0
    ws = 0
    if workspace is not None:
        ws = workspace.numel() * workspace.element_size()
    return _dev([(q, "q", _bf16(), rows), (k_pool, "k_pool", pool_t, pool_n), (v_pool, "v_pool", pool_t, pool_n),
                 (k_params, "k_params", (torch.float16,), par_n), (v_params, "v_params", (torch.float16,), par_n),
                 (out, "out", (torch.float32,), rows),
                 (workspace, "workspace", (workspace.dtype,) if workspace is not None else (), 0)]) + [ws]


PHASE_QPREP, PHASE_TILES, PHASE_COMBINE = 1, 2, 4


def paged_decode_attn_phases(shape, plan: DevicePlan, q, k_pool, v_pool, out, workspace, phases, layer=0, scale=None,
                             k_params=None, v_params=None):
    """The phases of paged_decode_attn selected by the bit mask ``phases``."""
    sh = make_shape(shape)
    if scale is None:
        scale = 1.0 / float(shape.head_dim) ** 0.5
    args = _decode_args(shape, plan, q, k_pool, v_pool, k_params, v_params, out, workspace)
    _check(lib().paged_decode_attn_phases(C.byref(sh), C.byref(plan.c), args[0], args[1], args[2], args[3], args[4],
                                          int(layer), float(scale), args[5], args[6], args[7], int(phases),
                                          _stream()))
    return out


def kv_rerotate(x, shift, rope_theta, out=None, out_dtype=None):
    """y = R(shift) x for x [rows, heads, d] (bf16 or float32), shift int32 [rows]."""
    import torch
    dt = {torch.bfloat16: KVP_BF16, torch.float32: KVP_F32}
    if x.dim() != 3:
        raise KvpError(KVP_EINVAL, "x: expected [rows, heads, head_dim]")
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    n = x.numel()
    px, po, ps = _dev([(x, "x", tuple(dt), n), (out, "out", tuple(dt), n), (shift, "shift", (torch.int32,), x.shape[0])])
    _check(lib().kv_rerotate(px, po, ps, x.shape[0], x.shape[1], x.shape[2],
                             float(rope_theta), dt[x.dtype], dt[out.dtype], _stream()))
    return out
