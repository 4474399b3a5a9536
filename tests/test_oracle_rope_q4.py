"""Pins of oracle/rope.py (RoPE offset compensation, INMS walkthrough sec. 2.3 /
3.2) and oracle/q4.py (groupwise Q4, Q4 KV paper summary sec. 2.1) against
closed forms and textbook identities."""
import numpy as np

from oracle import q4, rope
from workload import rng


def test_rotation_is_complex_multiplication():
    """Independent formulation: pair (x_i, x_{i+d/2}) as x_i + 1j*x_{i+d/2},
    rotated by exp(1j * delta * base**(-2i/d))."""
    r = np.random.default_rng(0)
    d, base = 16, 10000.0
    x = r.standard_normal((5, d))
    delta = np.array([0, 1, -7, 300, 12345])
    z = x[:, : d // 2] + 1j * x[:, d // 2:]
    freq = np.array([base ** (-2.0 * i / d) for i in range(d // 2)])
    zr = z * np.exp(1j * delta[:, None] * freq[None, :])
    want = np.concatenate([zr.real, zr.imag], axis=1)
    assert np.allclose(rope.rotate(x, delta, base), want, rtol=0, atol=1e-12)


def test_two_dim_direction():
    # a single pair with frequency 1: +delta turns (1, 0) towards (cos, sin)
    y = rope.rotate(np.array([1.0, 0.0]), 0.5, 1.0)
    assert np.allclose(y, [np.cos(0.5), np.sin(0.5)], atol=0)


def test_identity_zero_shift_exact():
    x = np.random.default_rng(1).standard_normal((3, 64))
    assert np.array_equal(rope.rotate(x, 0, 1e6), x)


def test_relative_identity_a_to_b():
    """R(b) R(a)^-1 x == R(b - a) x: the compensation depends only on b - a."""
    r = np.random.default_rng(2)
    x = r.standard_normal((8, 128))
    for a, b in [(0, 5), (100, 37), (4096, -12), (45000, 45100)]:
        back = rope.rotate(x, -a, 1e6)
        lhs = rope.rotate(back, b, 1e6)
        rhs = rope.rotate(x, b - a, 1e6)
        assert np.abs(lhs - rhs).max() < 1e-11


def test_inverse_and_pair_norms():
    r = np.random.default_rng(3)
    x = r.standard_normal((4, 128))
    y = rope.rotate(x, 777, 1e6)
    assert np.abs(rope.rotate(y, -777, 1e6) - x).max() < 1e-12
    n0 = x[:, :64] ** 2 + x[:, 64:] ** 2
    n1 = y[:, :64] ** 2 + y[:, 64:] ** 2
    assert np.abs(n0 - n1).max() < 1e-12


def test_scores_depend_on_relative_position_only():
    """(R(a) q) . (R(b) k) == q . R(b - a) k for every a, b (why the stored key can
    be moved by the difference alone)."""
    r = np.random.default_rng(4)
    q, k = r.standard_normal(64), r.standard_normal(64)
    ref = q @ rope.rotate(k, 13, 1e4)
    for a in [0, 5, 1000]:
        assert abs(rope.rotate(q, a, 1e4) @ rope.rotate(k, a + 13, 1e4) - ref) < 1e-10


# ---- Q4 ----------------------------------------------------------------------


def test_dequant_closed_form_and_nibble_order():
    d = 128
    codes = np.zeros((1, d // 2), np.uint8)
    codes[0, 0] = 0x5A   # element 0 -> 10 (low nibble), element 1 -> 5
    codes[0, 40] = 0xF0  # element 80 -> 0, element 81 -> 15
    params = np.array([[[0.5, -1.0], [0.25, 2.0]]], np.float16)
    x = q4.dequant(codes, params)
    assert x[0, 0] == 0.5 * 10 - 1.0
    assert x[0, 1] == 0.5 * 5 - 1.0
    assert x[0, 2] == -1.0
    assert x[0, 80] == 2.0
    assert x[0, 81] == 0.25 * 15 + 2.0


def test_encode_decode_error_bound_and_min():
    """The generator's encoding read back through the oracle: |x - x^| <= s/2 plus
    the fp16 roundings; codes in range; the group minimum decodes to z exactly."""
    bits = rng.bf16_tile((1, 2, 3, 4), 0, 0, (64, 128))
    x = rng.bf16_bits_to_f32(bits).astype(np.float64)
    codes, params = rng.q4_encode(bits)
    xr = q4.dequant(codes, params)
    s = params[..., 0].astype(np.float64)
    z = params[..., 1].astype(np.float64)
    mx = x.reshape(64, 2, 64).max(-1)
    err = np.abs(x - xr).reshape(64, 2, 64).max(-1)
    # rounding to a code is worth s/2; the fp16 scale may undershoot (max-min)/15,
    # leaving the top code short by at most 15 * |s16 - s32|
    s32 = (mx - x.reshape(64, 2, 64).min(-1)) / 15
    bound = s / 2 + 15 * np.abs(s - s32) + 1e-12
    assert (err <= bound).all()
    # the minimum decodes to z (code 0), which equals the bf16 minimum
    assert np.array_equal(xr.reshape(64, 2, 64).min(-1), z)
    assert np.array_equal(z, x.reshape(64, 2, 64).min(-1))


def test_q4_padding_rows_are_nan():
    bits = rng.bf16_tile((9, 9, 9, 9), 0, 0, (4, 128))
    bits[2:] = rng.BF16_NAN
    codes, params = rng.q4_encode(bits)
    assert np.isnan(params[2:].astype(np.float32)).all()
    assert (codes[2:] == 0).all()
    assert np.isfinite(params[:2].astype(np.float32)).all()
