"""Counter-based random numbers for the synthetic workload (host side).

Philox4x32-10 is implemented from its published definition (Salmon, Moraes,
Dror, Shaw: "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11): ten rounds of
two 32x32->64 multiplies (multipliers 0xD2511F53 and 0xCD9E8D57) with a Weyl key
schedule (0x9E3779B9, 0xBB67AE85).  The device filler in ``workload/csrc``
implements the same function; both sides must agree bit for bit, which a GPU
test checks.

Values are drawn so that host and device produce identical bits with integer
arithmetic only (no transcendental functions whose last bit could differ):

* ``ih_value``: an Irwin-Hall sum of the four bytes of one Philox word,
  centred and scaled by 7/1024 -> an approximately N(0, 1.02) value that is an
  exact float32; it is then rounded to bfloat16 (round-to-nearest-even).
* ``q4_encode``: 4-bit groupwise encoding (group of 64 consecutive head-dim
  elements, fp16 scale and fp16 zero = group minimum) of those bf16 values;
  this is how the persistent Q4 cache's blocks are produced.  Decoding is not
  here: it belongs to whoever reads the cache.

Nothing in this module computes any part of the attention method.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint32(0x9E3779B9)
PHILOX_W1 = np.uint32(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)

BF16_NAN = np.uint16(0x7FC0)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  All arguments broadcast; uint32 arrays out."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint32) for x in (c0, c1, c2, c3))
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    c0, c1, c2, c3 = (x.copy() for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint32).copy()
    k1 = np.asarray(k1, dtype=np.uint32).copy()
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0 = (k0 + PHILOX_W0).astype(np.uint32)
                k1 = (k1 + PHILOX_W1).astype(np.uint32)
            p0 = PHILOX_M0 * c0.astype(np.uint64)
            p1 = PHILOX_M1 * c2.astype(np.uint64)
            hi0 = (p0 >> np.uint64(32)).astype(np.uint32)
            lo0 = (p0 & MASK32).astype(np.uint32)
            hi1 = (p1 >> np.uint64(32)).astype(np.uint32)
            lo1 = (p1 & MASK32).astype(np.uint32)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def ih_value(word: np.ndarray) -> np.ndarray:
    """One Philox word -> exact float32 value (s - 510) * 7 / 1024."""
    w = np.asarray(word, dtype=np.uint32)
    s = ((w & 0xFF) + ((w >> 8) & 0xFF) + ((w >> 16) & 0xFF) + (w >> 24)).astype(np.int32) - 510
    return (s * 7).astype(np.float32) * np.float32(1.0 / 1024.0)


def seed_words(seed16: bytes) -> tuple[int, int, int, int]:
    """16-byte content seed -> four little-endian uint32 words."""
    a = np.frombuffer(seed16, dtype="<u4")
    return int(a[0]), int(a[1]), int(a[2]), int(a[3])


# Tensor selectors placed in the third Philox counter word (low byte); the layer
# index sits above it.  K, V and the query use disjoint streams.
SEL_K, SEL_V, SEL_Q = 0, 1, 2


def tile_words(seed: tuple[int, int, int, int], layer: int, sel: int, n_elem: int, e0: int = 0) -> np.ndarray:
    """Philox words for elements e0..e0+n_elem-1 of one tile (element e uses word
    e%4 of the Philox output for counter (e//4, seed[3], sel | layer<<8, seed[2])
    under key (seed[0], seed[1])).  e0 must be a multiple of 4."""
    assert e0 % 4 == 0
    nq = (n_elem + 3) // 4
    q = np.arange(e0 // 4, e0 // 4 + nq, dtype=np.uint32)
    s0, s1, s2, s3 = seed
    c2 = np.uint32((sel & 0xFF) | (layer << 8))
    o = philox4x32_10(q, np.uint32(s3), c2, np.uint32(s2), np.uint32(s0), np.uint32(s1))
    return np.stack(o, axis=1).reshape(-1)[:n_elem]


def bf16_range(seed, layer: int, sel: int, e0: int, n: int) -> np.ndarray:
    """bf16 bits of tile elements e0..e0+n-1 (e0 a multiple of 4)."""
    return f32_to_bf16_bits(ih_value(tile_words(seed, layer, sel, n, e0)))


def bf16_tile(seed, layer: int, sel: int, shape) -> np.ndarray:
    """A bf16 tile (as uint16 bits) of the given shape, row-major element order."""
    n = int(np.prod(shape))
    return f32_to_bf16_bits(ih_value(tile_words(seed, layer, sel, n))).reshape(shape)


def q4_encode(x_bf16_bits: np.ndarray, group: int = 64):
    """Groupwise 4-bit encoding along the last axis.

    Per group: s = fp16((max - min) / 15), z = fp16(min); code
    c = clamp(rint_even((x - z) / s), 0, 15) in float32 with the fp16-rounded
    s and z (c = 0 when s == 0).  Codes are packed two per byte, even element in
    the low nibble.  A group holding NaN (a padding slot) gets NaN scale and zero
    and all-zero codes.  Returns (codes uint8 [..., d/2], params float16 [..., d/64, 2]).
    """
    x = bf16_bits_to_f32(x_bf16_bits)
    d = x.shape[-1]
    assert d % group == 0
    xg = x.reshape(*x.shape[:-1], d // group, group)
    mn = xg.min(axis=-1)
    mx = xg.max(axis=-1)
    s16 = ((mx - mn) / np.float32(15.0)).astype(np.float32).astype(np.float16)
    z16 = mn.astype(np.float16)
    s = s16.astype(np.float32)[..., None]
    z = z16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.rint((xg - z) / s)
    c = np.where((s == 0) | ~np.isfinite(c), 0, np.clip(c, 0, 15)).astype(np.uint8).reshape(*x.shape[:-1], d)
    codes = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    params = np.stack([s16, z16], axis=-1)
    return codes, params
