"""The benchmark builds its caches on the device with torch casts; these CPU
tests check that those encoders give byte for byte the codes the oracle's
own encoders give (bf16 RNE, FP8 E4M3 with and without a per-row scale, OCP
MXFP4), so the oracle reads the same stored values the kernels read."""
import numpy as np
import pytest
import torch

import bench
import oracle as O


def _values(seed, rows, dim):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, dim)).astype(np.float32)
    x[:, 3] *= 8.0                                    # outlier channel
    x[1] = 0.0                                        # an all-zero row (and zero MX blocks)
    # exact E2M1 tie points and saturation in one MX block of row 2
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.5, -0.25, -0.75, -1.25, -1.75, -2.5,
                     -3.5, -5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, -6.0, 0.0, -0.0, 0.1, 0.3, 7.9, 0.7, 1.3, 2.7, 4.5],
                    np.float32)
    x[2, :32] = ties
    x[3, :dim] = np.float32(1e-30)                    # subnormal-scale block
    x[4, 5] = np.float32(500.0)                       # beyond E4M3 range unscaled
    return x


@pytest.mark.parametrize("dim", [128, 576])
def test_bf16_codes_match_oracle(dim):
    x = _values(1, 16, dim)
    got = bench.enc_bf16(torch, torch.from_numpy(x)).numpy()
    data, _ = O.alloc_rows(O.BF16, 16, dim, False)
    O.store_rows(O.BF16, data, None, 0, x)
    assert np.array_equal(got, data)


@pytest.mark.parametrize("dim", [128, 576])
def test_fp8_scaled_codes_match_oracle(dim):
    x = _values(2, 16, dim)
    got, s = bench.enc_fp8_scaled(torch, torch.from_numpy(x))
    data, scale = O.alloc_rows(O.FP8, 16, dim, True)
    O.store_rows(O.FP8, data, scale, 0, x)
    assert np.array_equal(s.numpy(), scale)
    assert np.array_equal(got.numpy(), data)


def test_fp8_raw_codes_match_oracle():
    x = _values(3, 16, 128)
    got = bench.enc_fp8_raw(torch, torch.from_numpy(x)).numpy()
    data, _ = O.alloc_rows(O.FP8, 16, 128, False)
    O.store_rows(O.FP8, data, None, 0, x)
    assert np.array_equal(got, data)


@pytest.mark.parametrize("dim", [128, 576])
def test_mxfp4_codes_match_oracle(dim):
    x = _values(4, 16, dim)
    got, sc = bench.enc_mxfp4(torch, torch.from_numpy(x))
    data, scale = O.alloc_rows(O.MXFP4, 16, dim, True)
    O.store_rows(O.MXFP4, data, scale, 0, x)
    assert np.array_equal(sc.numpy(), scale)
    assert np.array_equal(got.numpy(), data)


# --------------------------------------------------------------------------
# algorithmic bytes and flops per stage
# --------------------------------------------------------------------------

from long_context_compressed_append_amd import synth  # noqa: E402


def _decode_formulas(c, b_kv, b_ik, b_win):
    """Per-sequence byte counts of one decode row (one new token completing
    one entry), written out from the stage definitions."""
    N, E, H, D, HI, dI, k, w = c.max_entries, c.E, c.H, c.D, c.HI, c.dI, c.k, c.window
    sel = min(k, N) if HI else N
    index = N * b_ik + HI * dI * 2 + 4 * HI + 4 * N // E + 4 * N if HI else 0
    topk = 4 * N + 4 * k if HI else 0
    attn = sel * b_kv + (4 * k if HI else 0) + w * b_win + H * D * 2 + H * c.dv * 2 + 4 * H
    return index, topk, attn


@pytest.mark.parametrize("name,b_kv,b_ik,b_win", [("csa_64k", 1152, 256, 580), ("hca_1m", 1152, 0, 580),
                                                  ("lp_512k", 306, 128, 580)])
def test_stage_bytes_decode(name, b_kv, b_ik, b_win):
    c = synth.CONFIGS[name]
    w = bench.stage_work(c)
    index, topk, attn = _decode_formulas(c, b_kv, b_ik, b_win)
    assert w["index_logits"][0] == c.batch * index
    assert w["topk_select"][0] == c.batch * topk
    assert w["sparse_attn_fwd"][0] == c.batch * attn
    N = c.max_entries
    assert w["index_logits"][1] == c.batch * 2 * c.HI * c.dI * N
    assert w["sparse_attn_fwd"][1] == c.batch * 2 * c.H * (c.D + c.dv) * ((min(c.k, N) if c.HI else N) + 128)
    # compress: m-1 ring tokens + the new token read, one window slot and one entry per stream written
    tok = 2 * c.D + 4 + ((2 * c.dI + 4) if c.HI else 0)
    assert w["compress_append"][0] == c.batch * (c.m * tok + b_win + b_kv + b_ik)


def test_stage_bytes_prefill():
    c = synth.CONFIGS["prefill_8k"]
    w = bench.stage_work(c)
    rows = 8192
    sum_n = sum((p + 1) // 4 for p in range(122880, 131072))
    assert sum_n == 260_044_800
    keys = 131072 // 4
    assert w["index_logits"] == (keys * 256 + 512 * 4 + rows * (64 * 128 * 2 + 4 * 64) + 4 * sum_n,
                                 2 * 64 * 128 * sum_n)
    assert w["topk_select"][0] == 4 * sum_n + 4 * 2048 * rows
    # every entry of the sequence is selected by some row (unique bytes = all
    # entries); the windows of all rows span positions 122753 .. 131071
    attn = keys * 1152 + 4 * 2048 * rows + (131071 - 122753 + 1) * 1152 + rows * (64 * 576 * 4 + 256)
    assert w["sparse_attn_fwd"] == (attn, 2 * 64 * 1152 * (2048 + 128) * rows)
    assert w["compress_append"][0] == 8192 * ((1152 + 4 + 256 + 4) + 1152) + 2048 * (1152 + 256)
