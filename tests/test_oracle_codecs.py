"""Pins for the oracle's number formats (bf16, FP8 E4M3, E2M1/MXFP4).

Each codec is checked against something other than itself: torch's own
casts (a library routine), an exhaustive nearest-value search over every
code, and hand-computed blocks from the OCP MX rules."""
import numpy as np
import pytest
import torch

import oracle as O


def _torch_bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_encode_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-40, -1e-40, np.inf, -np.inf], np.float32),
    ]).astype(np.float32)
    # exact ties: low 16 bits = 0x8000 with odd and even kept parts
    bits = (rng.integers(0, 2**15, 5000, dtype=np.uint32) << 17 | np.uint32(0x8000)).astype(np.uint32)
    bits2 = bits | np.uint32(0x10000)
    x = np.concatenate([x, bits.view(np.float32), bits2.view(np.float32)])
    x = x[np.isfinite(x) | np.isinf(x)]
    got = O.bf16_encode(x)
    want = _torch_bf16_bits(x)
    assert np.array_equal(got, want)


def test_bf16_decode_is_exact_widening():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_decode(h)
    want = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def _fp8_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8_decode_all_codes_match_torch():
    got = O.fp8_decode(np.arange(256, dtype=np.uint8))
    want = _fp8_table()
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def _fp8_bruteforce(x):
    """Nearest finite E4M3 code, ties to the even code, saturating."""
    table = _fp8_table()
    finite = [c for c in range(256) if not np.isnan(table[c])]
    out = np.empty(len(x), np.uint8)
    for i, v in enumerate(x.astype(np.float64)):
        if v >= 448.0:
            out[i] = 0x7E; continue
        if v <= -448.0:
            out[i] = 0xFE; continue
        best = None
        for c in finite:
            if (table[c] == 0.0) and ((c & 0x80) != (0x80 if np.signbit(v) else 0)):
                continue       # signed zero follows the input's sign
            d = abs(table[c] - v)
            if best is None or d < bd or (d == bd and (c & 1) == 0 and (best & 1) == 1):
                best, bd = c, d
        out[i] = best
    return out


def test_fp8_encode_bruteforce_including_midpoints():
    table = _fp8_table()
    pos = np.sort(np.unique(table[:0x7F][~np.isnan(table[:0x7F])]))
    mids = (pos[1:] + pos[:-1]) / 2.0
    rng = np.random.default_rng(2)
    x = np.concatenate([pos, mids, pos * 1.0001, mids * 0.9999, mids * 1.0001,
                        rng.uniform(-500, 500, 3000), rng.standard_normal(3000) * 1e-2,
                        [0.0, -0.0, 449.0, 463.9, 464.0, 470.0, 1e6, -1e6]]).astype(np.float32)
    x = np.concatenate([x, -x])
    got = O.fp8_encode(x)
    want = _fp8_bruteforce(x)
    assert np.array_equal(got, want)


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * 60).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    got = O.fp8_encode(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


FP4_MAG = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP E2M1 value table


def test_fp4_decode_table():
    got = O.fp4_decode(np.arange(16, dtype=np.uint8))
    want = np.array(FP4_MAG + [-v for v in FP4_MAG])
    assert np.array_equal(got, want)


def test_fp4_encode_bruteforce():
    vals = np.array(FP4_MAG)
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(4)
    x = np.concatenate([vals, mids, mids + 1e-9, mids - 1e-9, rng.uniform(-8, 8, 5000), [6.5, 7.99, 100.0]])
    x = np.concatenate([x, -x])
    got = O.fp4_encode(x)
    for v, c in zip(x, got):
        a = min(abs(v), 6.0)
        d = np.abs(vals - a)
        cands = np.flatnonzero(d == d.min())
        want = cands[0] if len(cands) == 1 else [c2 for c2 in cands if c2 % 2 == 0][0]
        assert (c & 7) == want, (v, c)
        assert (c >> 3) == (1 if np.signbit(v) else 0)
    # explicit ties: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    ties = O.fp4_decode(O.fp4_encode(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])))
    assert list(ties) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]


def test_mx_scale_exponent_rule():
    # X = floor(log2(amax)) - 2, clamped to [-127, 127]; amax = 0 -> -127
    assert O.mx_scale_exp(1.0) == -2
    assert O.mx_scale_exp(4.0) == 0
    assert O.mx_scale_exp(7.99) == 0
    assert O.mx_scale_exp(8.0) == 1
    assert O.mx_scale_exp(0.75) == -3
    assert O.mx_scale_exp(0.0) == -127
    assert O.mx_scale_exp(2.0 ** -140) == -127
    assert O.mx_scale_exp(3.0e38) == 125


def test_mxfp4_rows_hand_blocks():
    dim = 64
    x = np.zeros((1, dim), np.float32)
    # block 0: amax = 4 exactly (power of two) -> X = 0, elements encode directly
    x[0, :8] = [4.0, -4.0, 0.25, 0.75, 1.25, 5.0, 6.0, -3.0]
    # block 1: amax = 7.5 -> X = 0, 7.5 saturates to 6; 0.3 -> 0.5 (nearest)
    x[0, 32:36] = [7.5, 0.3, -0.2, 2.9]
    data, scale = O.alloc_rows(O.MXFP4, 1, dim, True)
    O.store_rows(O.MXFP4, data, scale, 0, x)
    assert list(scale) == [127, 127]
    back = O.load_rows(O.MXFP4, data, scale, 0, 1, dim)[0]
    assert list(back[:8]) == [4.0, -4.0, 0.0, 1.0, 1.0, 4.0, 6.0, -3.0]
    assert list(back[32:36]) == [6.0, 0.5, 0.0, 3.0]
    # element 2i in the low nibble
    assert data[0] == (0b0110 | (0b1110 << 4))       # +4 low, -4 high
    # all-zero block -> scale byte 0 (X = -127), all codes zero
    assert np.all(back[8:32] == 0)


def test_mxfp4_scaled_block_and_error_bound():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, 576)).astype(np.float32) * np.float32(3.0)
    data, scale = O.alloc_rows(O.MXFP4, 200, 576, True)
    O.store_rows(O.MXFP4, data, scale, 0, x)
    back = O.load_rows(O.MXFP4, data, scale, 0, 200, 576)
    xb = x.reshape(200, 18, 32).astype(np.float64)
    amax = np.abs(xb).max(-1)
    X = np.floor(np.log2(amax)) - 2
    assert np.array_equal(scale.reshape(200, 18).astype(np.int64) - 127, X.astype(np.int64))
    # every element within half a quantum of its input, except saturated ones
    q = 2.0 ** X[..., None]
    err = np.abs(back.reshape(200, 18, 32) - xb)
    half = np.where(np.abs(xb) / q < 2, 0.25, np.where(np.abs(xb) / q < 4, 0.5, 1.0)) * q
    sat = np.abs(xb) / q > 6
    assert np.all((err <= half + 1e-12) | sat)
    assert np.all(np.abs(back.reshape(200, 18, 32)[sat]) == 6 * np.broadcast_to(q, sat.shape)[sat])


def test_fp8_rows_with_token_scale():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, 576)).astype(np.float32)
    x[3] = 0.0
    data, scale = O.alloc_rows(O.FP8, 50, 576, True)
    O.store_rows(O.FP8, data, scale, 0, x)
    amax = np.abs(x).max(1)
    s_want = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    assert np.array_equal(scale, s_want)
    codes = data.reshape(50, 576)
    want = _fp8_bruteforce((x / s_want[:, None]).astype(np.float32).ravel()).reshape(50, 576)
    assert np.array_equal(codes, want)
    # the row maximum maps to +-448 (code 0x7E / 0xFE)
    i = np.abs(x).argmax(1)
    assert np.all((codes[np.arange(50), i] & 0x7F)[amax > 0] == 0x7E)
    back = O.load_rows(O.FP8, data, scale, 0, 50, 576)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 + s_want[:, None] * 2.0 ** -10)


def test_bf16_rows_roundtrip_and_raw_fp8_rows():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((10, 128)).astype(np.float32)
    d, s = O.alloc_rows(O.BF16, 10, 128, False)
    O.store_rows(O.BF16, d, s, 0, x)
    assert np.array_equal(d.view(np.uint16).reshape(10, 128), _torch_bf16_bits(x).reshape(10, 128))
    d8, s8 = O.alloc_rows(O.FP8, 10, 128, False)
    assert s8 is None
    O.store_rows(O.FP8, d8, None, 0, x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(d8.reshape(10, 128), want)
