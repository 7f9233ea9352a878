"""Pins of the oracle's rotary position embedding (applied to decoded keys,
which the cache holds before the rotation: 163.com article, section 5,
implementation details) and of the 3-D position table the tests feed it.

The rotation is checked against what the mathematics fixes, not against a
retyped copy of itself: angle zero is the identity, a quarter turn swaps the
pair with a sign, and every output lies within the fp32 rounding bound of the
complex product (a + i b)(cos + i sin) taken in complex128."""
import numpy as np

import oracle
import synthkv

U = 2.0 ** -24   # unit roundoff of fp32


def _rows(rng, n, d):
    return (rng.standard_normal((n, d)) * rng.lognormal(0, 2, (n, 1))).astype(np.float32)


def _table(rng, n, d):
    ang = rng.uniform(-np.pi, np.pi, (n, d // 2))
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def test_zero_angle_is_the_identity():
    rng = np.random.default_rng(1)
    y = _rows(rng, 50, 128)
    t = np.zeros((50, 64, 2), np.float32)
    t[..., 0] = 1.0
    np.testing.assert_array_equal(oracle.rope_rotate(y, t).view(np.uint32), y.view(np.uint32))


def test_quarter_turn_maps_a_b_to_minus_b_a():
    rng = np.random.default_rng(2)
    y = _rows(rng, 40, 64)
    t = np.zeros((40, 32, 2), np.float32)
    t[..., 1] = 1.0
    r = oracle.rope_rotate(y, t)
    np.testing.assert_array_equal(r[:, 0::2], -y[:, 1::2])
    np.testing.assert_array_equal(r[:, 1::2], y[:, 0::2])
    # a half turn negates; three quarter turns undo one
    t2 = np.zeros_like(t)
    t2[..., 0] = -1.0
    np.testing.assert_array_equal(oracle.rope_rotate(y, t2), -y)
    t3 = np.zeros_like(t)
    t3[..., 1] = -1.0
    np.testing.assert_array_equal(oracle.rope_rotate(r, t3), y)


def test_within_rounding_of_the_complex_product():
    """Each output is fl(fl(p) -/+ fl(q)) for exact products p, q, so it differs
    from the exact p -/+ q by at most u (|p| + |q|) (1 + u) + u |p -/+ q|.  A
    wrong sign, a swapped operand or the half-split pair layout misses this by
    orders of magnitude."""
    rng = np.random.default_rng(3)
    for d in (64, 128):
        y = _rows(rng, 300, d)
        t = _table(rng, 300, d)
        r = oracle.rope_rotate(y, t).astype(np.float64)
        z = (y[:, 0::2].astype(np.float64) + 1j * y[:, 1::2]) * (t[..., 0].astype(np.float64) + 1j * t[..., 1])
        a, b = y[:, 0::2].astype(np.float64), y[:, 1::2].astype(np.float64)
        c, s = t[..., 0].astype(np.float64), t[..., 1].astype(np.float64)
        bound_re = U * (np.abs(a * c) + np.abs(b * s)) * (1 + U) + U * np.abs(z.real)
        bound_im = U * (np.abs(a * s) + np.abs(b * c)) * (1 + U) + U * np.abs(z.imag)
        assert (np.abs(r[:, 0::2] - z.real) <= bound_re).all()
        assert (np.abs(r[:, 1::2] - z.imag) <= bound_im).all()


def test_decode_chunk_rotates_the_first_heads_before_rounding():
    """Keys rotated, values left alone, one rounding to bf16 after the
    rotation (rounding before it changes some outputs)."""
    rng = np.random.default_rng(4)
    H, N, d, K, G = 3, 64, 64, 8, 16
    codes = rng.integers(0, 256, (H, N, d // 4), dtype=np.uint8)
    scales = np.full((H, N, d // G), 0x38, np.uint8)          # scale 1.0
    asg = rng.integers(0, K, (1, H, N), dtype=np.uint8)
    cent = oracle.bf16_round(rng.standard_normal((1, H, K, d)) * 4).astype(np.float32)
    t = _table(rng, N, d)
    plain = oracle.decode_chunk(codes, scales, asg, cent, G, "f32")
    rot = oracle.decode_chunk(codes, scales, asg, cent, G, "bf16", rope=t, rope_heads=2)
    for h in range(2):
        np.testing.assert_array_equal(rot[h], oracle.bf16_round(oracle.rope_rotate(plain[h], t)))
    np.testing.assert_array_equal(rot[2], oracle.bf16_round(plain[2]))
    twice = oracle.bf16_round(oracle.rope_rotate(oracle.bf16_round(plain[0]).astype(np.float32), t))
    assert (twice != rot[0]).any()


def test_3d_table_is_a_rotation_by_position():
    """cos^2 + sin^2 = 1; token 0 is unrotated; along each axis the angle grows
    linearly with the position, so the table at position m + n is the rotation
    at m composed with the one at n (angle addition)."""
    p = synthkv.PRESETS[3]
    rows, cols = p.grid
    ft = rows * cols
    t = synthkv.rope_table(p, 0, 3 * ft).astype(np.float64)
    assert np.abs(t[..., 0] ** 2 + t[..., 1] ** 2 - 1).max() < 1e-6
    np.testing.assert_array_equal(t[0, :, 0], 1.0)
    np.testing.assert_array_equal(t[0, :, 1], 0.0)
    z = t[..., 0] + 1j * t[..., 1]
    gf, gr, gc = synthkv.rope_axis_pairs(p.d)
    assert gf + gr + gc == p.d // 2
    # frame 2 = frame 1 twice; row 4 = row 1 then row 3; column 7 = 3 + 4
    assert np.abs(z[2 * ft] - z[ft] ** 2).max() < 1e-6
    assert np.abs(z[4 * cols] - z[cols] * z[3 * cols]).max() < 1e-6
    assert np.abs(z[7] - z[3] * z[4]).max() < 1e-6
    # each axis moves only its own pairs
    assert np.abs(z[ft, gf:] - 1).max() == 0
    assert np.abs(z[cols, :gf] - 1).max() == 0 and np.abs(z[cols, gf + gr:] - 1).max() == 0
    assert np.abs(z[1, :gf + gr] - 1).max() == 0
    # a table for a later range is the same rows
    np.testing.assert_array_equal(synthkv.rope_table(p, 100, 200), t[100:200].astype(np.float32))
