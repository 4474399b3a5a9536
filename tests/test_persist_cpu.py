"""Persistent Q4 pool files on the CPU: the image size, the file round trip, the
format against the safetensors library (it reads our files; we read its files),
the agent namespace and the error paths.  No GPU: images are numpy arrays."""
import os

import numpy as np
import pytest
import safetensors
import safetensors.numpy as stn

from oracle import persist as ops
from shared_paged_kv_amd import _lib as K
from workload import spec


def _shape(L=1, H=8, B=256, d=128):
    return spec.Shape(L, 4 * H, H, d, B, spec.Q4G64, 1e4)


def _pools(g, sh, P):
    L, H, B, d = sh.n_layers, sh.n_kv_heads, sh.block_tokens, sh.head_dim
    kc = g.integers(0, 256, (L, P, H, B, d // 2), dtype=np.uint8)
    vc = g.integers(0, 256, (L, P, H, B, d // 2), dtype=np.uint8)
    kp = g.standard_normal((L, P, H, B, d // 64, 2)).astype(np.float16)
    vp = g.standard_normal((L, P, H, B, d // 64, 2)).astype(np.float16)
    return kc, vc, kp, vp


def test_image_bytes_closed_form():
    sh = _shape()
    # per block and layer: 2 x (8 heads x 256 tokens x 64 code bytes) + 2 x (8 x 256 x 2 groups x (s, z) x 2 bytes)
    per = 2 * 8 * 256 * 64 + 2 * 8 * 256 * 2 * 2 * 2
    assert per == 294912
    assert K.q4_image_bytes(sh, 32) == 32 * per
    assert K.q4_image_bytes(_shape(L=48), 3) == 48 * 3 * per
    # 0.28125 of the bf16 bytes of the same block (Q4 KV paper summary, sec. 2.1)
    assert per / (2 * 8 * 256 * 128 * 2) == 0.28125
    with pytest.raises(K.KvpError):
        K.q4_image_bytes(spec.Shape(1, 32, 8, 128, 256, spec.BF16, 1e4), 1)


@pytest.mark.parametrize("L,n", [(1, 3), (4, 9)])
def test_round_trip_and_safetensors_reads_our_file(tmp_path, L, n):
    g = np.random.default_rng(L * 10 + n)
    sh = _shape(L=L)
    P = n + 5
    pools = _pools(g, sh, P)
    ids = list(g.permutation(P)[:n])
    img = np.frombuffer(ops.q4_image(*pools, ids), np.uint8).copy()
    assert img.nbytes == K.q4_image_bytes(sh, n)
    ntok = g.integers(0, sh.block_tokens + 1, n).astype(np.int32)
    path = tmp_path / "agent7.safetensors"
    K.q4_save_file(sh, path, "agent-7", img, ntok)
    # our reader
    back = np.zeros_like(img)
    got_n, got_nt = K.q4_load_file(sh, path, "agent-7", back)
    assert got_n == n and np.array_equal(got_nt, ntok) and np.array_equal(back, img)
    assert K.q4_load_file(sh, path) == n
    # the safetensors library
    t = stn.load_file(str(path))
    names = ["k_codes", "v_codes", "k_params", "v_params"]
    assert sorted(t) == sorted(names + ["ntok"])
    for name, pool in zip(names, pools):
        assert np.array_equal(t[name], np.stack([pool[:, i] for i in ids], 1))
    assert np.array_equal(t["ntok"], ntok)
    with safetensors.safe_open(str(path), "np") as f:
        md = f.metadata()
    assert md["agent"] == "agent-7" and md["format"] == "kvpool-q4g64"
    assert md["n_layers"] == str(L) and md["block_tokens"] == "256"
    assert (os.path.getsize(path) - img.nbytes - 4 * n) % 8 == 0


def test_we_read_a_file_the_library_wrote(tmp_path):
    """Tensors in the library's own order and alignment, extra tensors and
    metadata: our reader takes the named tensors wherever they are."""
    g = np.random.default_rng(3)
    sh = _shape(L=2, H=2, B=16, d=64)
    n = 5
    kc, vc, kp, vp = _pools(g, sh, n)
    ntok = np.array([16, 1, 0, 9, 16], np.int32)
    path = str(tmp_path / "lib.safetensors")
    stn.save_file({"v_params": vp, "zzz_extra": np.arange(7, dtype=np.float32), "k_codes": kc, "ntok": ntok,
                   "v_codes": vc, "k_params": kp}, path, metadata={"agent": "a1", "other": "x"})
    want = np.frombuffer(ops.q4_image(kc, vc, kp, vp, range(n)), np.uint8)
    img = np.zeros(K.q4_image_bytes(sh, n), np.uint8)
    got_n, got_nt = K.q4_load_file(sh, path, "a1", img)
    assert got_n == n and np.array_equal(got_nt, ntok) and np.array_equal(img, want)


def test_namespace_and_errors(tmp_path):
    g = np.random.default_rng(4)
    sh = _shape(L=1, H=2, B=16, d=64)
    n = 3
    pools = _pools(g, sh, n)
    img = np.frombuffer(ops.q4_image(*pools, range(n)), np.uint8).copy()
    ntok = np.array([16, 16, 4], np.int32)
    path = tmp_path / "a.safetensors"
    K.q4_save_file(sh, path, "alice", img, ntok)

    def code(fn):
        with pytest.raises(K.KvpError) as e:
            fn()
        return e.value.code

    buf = np.zeros_like(img)
    # another agent's file
    assert code(lambda: K.q4_load_file(sh, path, "bob", buf)) == K.KVP_EINVAL
    assert not buf.any()
    # another shape: tensors do not match
    assert code(lambda: K.q4_load_file(_shape(L=1, H=4, B=16, d=64), path)) == K.KVP_EINVAL
    assert code(lambda: K.q4_load_file(_shape(L=2, H=2, B=16, d=64), path)) == K.KVP_EINVAL
    # not a Q4 shape
    assert code(lambda: K.q4_load_file(spec.Shape(1, 4, 2, 64, 16, spec.BF16, 1e4), path)) == K.KVP_EINVAL
    # missing file, truncated file, garbage header
    assert code(lambda: K.q4_load_file(sh, tmp_path / "none.safetensors")) == K.KVP_EIO
    raw = open(path, "rb").read()
    (tmp_path / "trunc.safetensors").write_bytes(raw[: len(raw) - 10])
    assert code(lambda: K.q4_load_file(sh, tmp_path / "trunc.safetensors")) == K.KVP_EIO
    hl = int.from_bytes(raw[:8], "little")
    bad = raw[:8] + b"{" + b" " * (hl - 1) + raw[8 + hl:]
    (tmp_path / "json.safetensors").write_bytes(bad)
    assert code(lambda: K.q4_load_file(sh, tmp_path / "json.safetensors")) == K.KVP_EIO
    (tmp_path / "len.safetensors").write_bytes((10 ** 12).to_bytes(8, "little") + raw[8:])
    assert code(lambda: K.q4_load_file(sh, tmp_path / "len.safetensors")) == K.KVP_EIO
    # a missing tensor, a wrong dtype, ntok out of range (files written by the library)
    kc, vc, kp, vp = pools
    p2 = str(tmp_path / "miss.safetensors")
    stn.save_file({"k_codes": kc, "v_codes": vc, "k_params": kp, "ntok": ntok}, p2)
    assert code(lambda: K.q4_load_file(sh, p2)) == K.KVP_EINVAL
    stn.save_file({"k_codes": kc, "v_codes": vc, "k_params": kp, "v_params": vp.astype(np.float32), "ntok": ntok}, p2)
    assert code(lambda: K.q4_load_file(sh, p2)) == K.KVP_EINVAL
    stn.save_file({"k_codes": kc, "v_codes": vc, "k_params": kp, "v_params": vp,
                   "ntok": np.array([16, 17, 0], np.int32)}, p2)
    buf2 = np.zeros_like(img)
    assert code(lambda: K.q4_load_file(sh, p2, None, buf2)) == K.KVP_EINVAL
    assert not buf2.any()
    # bad arguments to save
    assert code(lambda: K.q4_save_file(sh, tmp_path / "b.safetensors", 'x"y', img, ntok)) == K.KVP_EINVAL
    assert code(lambda: K.q4_save_file(sh, tmp_path / "b.safetensors", "x", img, np.array([16, 16, 99], np.int32))) \
        == K.KVP_EINVAL
    assert code(lambda: K.q4_save_file(sh, tmp_path / "nodir" / "b.safetensors", "x", img, ntok)) == K.KVP_EIO
    # a too small image: only the count comes back
    small = np.zeros(img.nbytes - 1, np.uint8)
    with pytest.raises(K.KvpError):
        K.q4_load_file(sh, path, "alice", small)
    assert not small.any()


def test_oracle_scatter_inverts_gather():
    g = np.random.default_rng(6)
    sh = _shape(L=2, H=2, B=16, d=64)
    pools = _pools(g, sh, 10)
    ids = [7, 2, 3, 4, 9]
    img = ops.q4_image(*pools, ids)
    blank = [np.zeros_like(p) for p in pools]
    back = ops.scatter(blank, img, ids)
    for p, b in zip(pools, back):
        assert np.array_equal(b[:, ids], p[:, ids])
        others = [i for i in range(10) if i not in ids]
        assert not b[:, others].any()


def test_gather_scatter_argument_errors_without_launch():
    import ctypes as C
    sh = K.make_shape(_shape(L=1, H=2, B=16, d=64))
    L = K.lib()
    one = C.c_void_p(1)
    P32 = C.POINTER(C.c_int32)
    ids = (C.c_int32 * 2)(0, 5)
    idp = C.cast(ids, P32)
    assert L.kv_q4_gather(C.byref(sh), one, one, one, one, 5, idp, 2, one, None) == K.KVP_EINVAL  # id 5 >= 5
    assert L.kv_q4_gather(C.byref(sh), one, one, one, one, 8, None, 2, one, None) == K.KVP_EINVAL
    assert L.kv_q4_gather(C.byref(sh), one, None, one, one, 8, idp, 2, one, None) == K.KVP_EINVAL
    assert L.kv_q4_gather(C.byref(sh), one, one, one, one, 8, idp, 2, None, None) == K.KVP_EINVAL
    assert L.kv_q4_scatter(C.byref(sh), one, -1, one, one, one, one, 8, idp, None) == K.KVP_EINVAL
    assert L.kv_q4_scatter(C.byref(sh), one, 2, one, one, one, one, 0, idp, None) == K.KVP_EINVAL
    bf = K.make_shape(spec.Shape(1, 4, 2, 64, 16, spec.BF16, 1e4))
    assert L.kv_q4_scatter(C.byref(bf), one, 2, one, one, one, one, 8, idp, None) == K.KVP_EINVAL
    assert L.kv_q4_gather(C.byref(sh), one, one, one, one, 8, idp, 0, one, None) == K.KVP_OK  # nothing to do


def test_reader_survives_mutated_files(tmp_path):
    """Seeded mutations of a valid file -- truncations at every region, flipped
    and overwritten header bytes, forged length prefixes, garbage headers,
    trailing bytes -- are either read as a file (when the mutation left a valid
    one) or refused with KVP_EIO / KVP_EINVAL; the reader never writes the
    image of a refused file.  Under the sanitizer build
    (tests/test_host_sanitized.py) any out-of-bounds access shows up here."""
    g = np.random.default_rng(11)
    sh = _shape(L=1, H=2, B=16, d=64)
    n = 3
    pools = _pools(g, sh, n)
    img = np.frombuffer(ops.q4_image(*pools, range(n)), np.uint8).copy()
    ntok = np.array([16, 9, 1], np.int32)
    path = tmp_path / "ok.safetensors"
    K.q4_save_file(sh, path, "agent-3", img, ntok)
    raw = bytearray(open(path, "rb").read())
    hl = int.from_bytes(raw[:8], "little")
    mutants = []
    for cut in sorted(set(g.integers(0, len(raw), 60).tolist()) | {0, 1, 7, 8, 9, 8 + hl - 1, 8 + hl, len(raw) - 1}):
        mutants.append(bytes(raw[:cut]))
    for _ in range(120):
        m = bytearray(raw)
        for _ in range(int(g.integers(1, 6))):
            i = int(g.integers(0, 8 + hl))
            m[i] = int(g.integers(0, 256)) if g.random() < 0.5 else m[i] ^ (1 << int(g.integers(0, 8)))
        mutants.append(bytes(m))
    for v in [0, 1, 2, hl - 1, hl + 1, len(raw) - 8, len(raw) - 7, len(raw), 2 ** 31, 2 ** 63 - 1, 2 ** 64 - 1]:
        mutants.append(int(v % 2 ** 64).to_bytes(8, "little") + bytes(raw[8:]))
    for _ in range(40):
        k = int(g.integers(0, 2 * hl))
        junk = bytes(g.integers(0, 256, k, dtype=np.uint8)) if g.random() < 0.5 else \
            bytes(g.choice(list(b'{}[]":,0123456789.-eE truefalsnul\\'), k))
        mutants.append(len(junk).to_bytes(8, "little") + junk + bytes(raw[8 + hl:]))
    mutants.append(bytes(raw) + bytes(g.integers(0, 256, 37, dtype=np.uint8)))
    ok = refused = 0
    mp = tmp_path / "m.safetensors"
    for i, m in enumerate(mutants):
        mp.write_bytes(m)
        buf = np.zeros_like(img)
        try:
            got_n, got_nt = K.q4_load_file(sh, mp, None, buf)
        except K.KvpError as e:
            assert e.code in (K.KVP_EIO, K.KVP_EINVAL), (i, e)
            assert not buf.any(), i
            refused += 1
            continue
        # accepted: a well-formed file of this shape, ntok in range
        assert got_n == len(got_nt) and ((got_nt >= 0) & (got_nt <= sh.block_tokens)).all(), i
        ok += 1
    assert refused > len(mutants) // 2 and ok + refused == len(mutants)
