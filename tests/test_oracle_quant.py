"""Pins for the oracle's FP8 query quantisation (orc_quantize_fp8_rows): one
power-of-two scale per row, X = floor(log2 max|x|) - 7, codes = RNE E4M3 of
x / 2^X.

Checked against: the exponent rule (the row maximum lands in [128, 256)),
torch's float8_e4m3fn cast of x / 2^X (an independent RNE implementation,
exact division by a power of two), scale covariance (x * 2^k gives X + k
and the same codes), the element-wise error bound of the format, and the
zero row."""
import numpy as np
import torch

import oracle as O


def _rows(seed, n=64, dim=128):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, dim)).astype(np.float32)
    mags = 2.0 ** rng.integers(-30, 30, n)
    x *= mags[:, None].astype(np.float32)
    x[0, 5] = 1.0                                           # an exact power of two as the maximum
    x[0, :5] = 0.0
    x[0, 6:] = np.clip(x[0, 6:], -0.9, 0.9)
    return x


def test_row_maximum_lands_in_128_256():
    x = _rows(1)
    c, X = O.quantize_fp8_rows(x)
    top = np.abs(O.fp8_decode(c)).max(axis=1)
    assert np.all(top >= 128.0) and np.all(top < 256.0 + 16.0)   # RNE may round the top up by a quantum
    amax = np.abs(x).max(axis=1).astype(np.float64)
    assert np.all(amax >= 128.0 * 2.0 ** X) and np.all(amax < 256.0 * 2.0 ** X)
    assert X[0] == -7                                       # max 1.0 = 2^0


def test_codes_equal_torch_cast_of_scaled_row():
    x = _rows(2)
    c, X = O.quantize_fp8_rows(x)
    scaled = torch.from_numpy(x.astype(np.float64) * 2.0 ** (-X[:, None].astype(np.float64))).to(torch.float32)
    want = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(c, want)


def test_scale_covariance():
    x = _rows(3)
    c, X = O.quantize_fp8_rows(x)
    for k in (-5, 3, 11):
        c2, X2 = O.quantize_fp8_rows((x.astype(np.float64) * 2.0 ** k).astype(np.float32))
        assert np.array_equal(c2, c)
        assert np.array_equal(X2, X + k)


def test_elementwise_error_bound():
    """|x - decode(code) 2^X| <= max(2^-4 |x|, 2^(X-10)): half a quantum of
    the element's binade (3 mantissa bits), or of the subnormal binade."""
    x = _rows(4)
    c, X = O.quantize_fp8_rows(x)
    s = 2.0 ** X[:, None].astype(np.float64)
    err = np.abs(x - O.fp8_decode(c) * s)
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s)
    assert np.all(err <= bound)


def test_zero_row():
    c, X = O.quantize_fp8_rows(np.zeros((2, 64), np.float32))
    assert np.all(c == 0) and np.all(X == -127)
