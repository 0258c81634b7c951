"""Pins for the oracle's rotary embedding (orc_rope).

The pages name RoPE on the shared KV vectors and its inverse on the output
but fix no convention; the oracle takes it as parameters (pairing, base or an
explicit frequency table, the slice of dims).  Pinned by what any rotary
embedding must satisfy, not by retyping it:

* position 0 and dims outside [off, off + rd) are left exactly as they are;
* the direction and the unit of the angle: (1, 0) at angle 1 rad goes to
  (cos 1, sin 1), printed below as decimal constants;
* rotations compose and the inverse undoes the forward (with power-of-two
  frequencies, so every fp32 angle is exact);
* the relative-position property: <R(p) q, R(s) k> = <R(p - s) q, k>;
* each pair's norm is kept;
* the frequencies recovered from the output (atan2 at position 1) form the
  geometric progression 1, theta^(-2/rd), theta^(-4/rd), ...;
* the half-split pairing is the interleaved one under a permutation of dims.
"""
import numpy as np

import oracle as O

COS1, SIN1 = 0.5403023058681398, 0.8414709848078965


def _x(seed, rows=5, heads=3, dim=24):
    return np.random.default_rng(seed).standard_normal((rows, heads, dim))


def _pow2_freq(rd):
    """Frequencies 1, 1/4, 1/16, ... (exact angles for integer positions)."""
    return (2.0 ** (-2.0 * np.arange(rd // 2))).astype(np.float32)


def test_position_zero_and_outside_slice_unchanged():
    x = _x(1)
    pos = np.array([0, 7, 100, 3, 12345])
    for pairing in (0, 1):
        y = O.rope(x, pos, off=4, rd=16, pairing=pairing)
        assert np.array_equal(y[0], x[0])
        assert np.array_equal(y[:, :, :4], x[:, :, :4])
        assert np.array_equal(y[:, :, 20:], x[:, :, 20:])
        assert not np.allclose(y[1:, :, 4:20], x[1:, :, 4:20])


def test_direction_and_unit_of_the_angle():
    x = np.zeros((1, 1, 2))
    x[0, 0, 0] = 1.0
    y = O.rope(x, [1], off=0, rd=2)                        # one pair, frequency theta^0 = 1
    assert abs(y[0, 0, 0] - COS1) < 1e-15 and abs(y[0, 0, 1] - SIN1) < 1e-15
    z = O.rope(x, [1], off=0, rd=2, inverse=True)
    assert abs(z[0, 0, 0] - COS1) < 1e-15 and abs(z[0, 0, 1] + SIN1) < 1e-15


def test_composition_and_inverse():
    x = _x(2, dim=16)
    fr = _pow2_freq(16)
    p = np.array([3, 17, 250, 1, 64])
    s = np.array([5, 2, 31, 1000, 0])
    for pairing in (0, 1):
        two = O.rope(O.rope(x, s, 0, 16, freq=fr, pairing=pairing), p, 0, 16, freq=fr, pairing=pairing)
        one = O.rope(x, p + s, 0, 16, freq=fr, pairing=pairing)
        assert np.abs(two - one).max() < 1e-12
        back = O.rope(O.rope(x, p, 0, 16, freq=fr, pairing=pairing), p, 0, 16, freq=fr, pairing=pairing,
                      inverse=True)
        assert np.abs(back - x).max() < 1e-13
    # the inverse with the default (non power-of-two) frequencies too
    q = np.array([1, 4095, 65535, 999999, 7])
    back = O.rope(O.rope(x, q, 0, 16), q, 0, 16, inverse=True)
    assert np.abs(back - x).max() < 1e-13


def test_relative_position_property():
    rng = np.random.default_rng(3)
    rd = 32
    fr = _pow2_freq(rd)
    q = rng.standard_normal((1, 1, rd))
    k = rng.standard_normal((1, 1, rd))
    for p, s in ((9, 4), (100, 37), (5, 5), (2, 30)):
        lhs = float(np.sum(O.rope(q, [p], 0, rd, freq=fr) * O.rope(k, [s], 0, rd, freq=fr)))
        if p >= s:
            rhs = float(np.sum(O.rope(q, [p - s], 0, rd, freq=fr) * k))
        else:
            rhs = float(np.sum(q * O.rope(k, [s - p], 0, rd, freq=fr)))
        assert abs(lhs - rhs) < 1e-12, (p, s)


def test_pair_norms_kept():
    x = _x(4, dim=32)
    pos = np.array([1, 1000, 123456, 7, 1 << 20])
    for pairing in (0, 1):
        y = O.rope(x, pos, 0, 32, pairing=pairing)
        if pairing == 0:
            n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
            n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
        else:
            n0 = x[..., :16] ** 2 + x[..., 16:] ** 2
            n1 = y[..., :16] ** 2 + y[..., 16:] ** 2
        assert np.abs(n0 - n1).max() < 1e-12


def test_frequencies_form_the_geometric_progression():
    rd, theta = 64, 10000.0
    x = np.zeros((1, 1, rd))
    x[0, 0, 0::2] = 1.0
    y = O.rope(x, [1], 0, rd, theta=theta)
    f = np.arctan2(y[0, 0, 1::2], y[0, 0, 0::2])          # angle at position 1 (all < pi)
    assert f[0] == 1.0 or abs(f[0] - 1.0) < 1e-15
    want = theta ** (-2.0 * np.arange(rd // 2) / rd)
    assert np.all(np.abs(f / want - 1.0) < 2.0 ** -23)    # fp32 frequencies
    assert abs(f[-1] * theta ** (2.0 * (rd // 2 - 1) / rd) - 1.0) < 2.0 ** -23


def test_half_split_is_interleaved_under_a_permutation():
    x = _x(5, dim=16)
    pos = np.array([2, 77, 4096, 31, 500000])
    perm = np.concatenate([np.arange(0, 16, 2), np.arange(1, 16, 2)])   # interleaved -> half split
    a = O.rope(x, pos, 0, 16, pairing=0)
    b = O.rope(x[..., perm], pos, 0, 16, pairing=1)
    assert np.array_equal(a[..., perm], b)
