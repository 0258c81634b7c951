"""Comparison rules between the device library and the oracle.

* Stored codes written by compress_append: the device's fp32 aggregate
  differs from the oracle's fp64 aggregate (rounded to fp32) by a few fp32
  ulps, so a code may differ only where that value sits next to a rounding
  boundary.  Rule: every device code must decode to a correct rounding of
  the oracle's fp32 value (within half a quantum, plus 1% slack), and at
  least 99.9% of the codes must be identical.  Quanta are computed here
  from the format definitions, independently of both codecs.
* Indexer logits: |gpu - oracle| <= 2e-5 * sum_h w_h sum_d |q_hd k_d| (a
  forward error bound of fp32 summation over ~200 terms).
* Top-k on identical logits: identical index lists.
* End-to-end top-k: with L_k the oracle's k-th largest logit and
  tau = 1e-3 |L_k|, the device set holds every entry above L_k + tau and
  none below L_k - tau, and has min(k, n) entries.
* Attention outputs: max-abs 2e-2, mean-abs 2e-3 and relative L2 1e-2 for
  bf16/FP8 paths, max-abs 5e-2 for MXFP4 caches, on the raw fp32 outputs;
  fp32 workloads max-abs 1e-5.  Tests of the bf16-output variant (and only
  those) pass out_bf16=True, which discounts the output's own rounding, half
  a bf16 ulp of the value: at the csa outlier channels' magnitudes (16-32)
  that is up to 0.0625, beyond the 2e-2 bound by itself.
"""
import numpy as np

import oracle as O


def ulp_bf16(x):
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return 2.0 ** (e - 7)


def quantum_fp8(x):
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6)
    return 2.0 ** (e - 3)


def check_correct_rounding(dtype, got_deq, exact32, eps, got_codes=None, want_codes=None, dim=None,
                           got_scale=None):
    """got_deq: device values decoded (float64); exact32: the oracle's value
    before encoding, rounded to fp32; eps: bound on the device's own fp32
    error for each value (the stored code must be a correct rounding of some
    value within eps of exact32)."""
    x = exact32.astype(np.float64)
    eps = np.broadcast_to(np.asarray(eps, np.float64), x.shape)
    ax = np.abs(x)
    if dtype == O.BF16:
        bad = np.abs(got_deq - x) > 0.5 * ulp_bf16(ax + eps) + eps
    elif dtype == O.FP8:
        sat = ax - eps >= 448.0
        near = ax + eps >= 448.0
        ok = np.abs(got_deq - x) <= 0.5 * quantum_fp8(ax + eps) + eps
        ok |= near & (np.abs(got_deq) == 448.0)
        bad = np.where(sat, got_deq != np.sign(x) * 448.0, ~ok)
    elif dtype == O.MXFP4:
        xb = x.reshape(-1, dim // 32, 32)
        eb = eps.reshape(xb.shape)
        lo = np.maximum(np.abs(xb) - eb, 0).max(-1)
        hi = (np.abs(xb) + eb).max(-1)

        def sexp(a):
            return np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))) - 2, -127)
        Xg = got_scale.reshape(-1, dim // 32).astype(np.int64) - 127
        scale_ok = (Xg == sexp(lo)) | (Xg == sexp(hi))
        assert scale_ok.all(), "MXFP4 block scales differ away from a power-of-two boundary"
        s = 2.0 ** Xg[..., None]
        v, ev = np.abs(xb) / s, eb / s
        q = np.where(v + ev < 2, 0.5, np.where(v + ev < 4, 1.0, 2.0)) * s
        gd = got_deq.reshape(xb.shape)
        ok = np.abs(gd - xb) <= 0.5 * q + eb
        ok |= (v + ev >= 6) & (np.abs(gd) == 6 * s) & (np.sign(gd) == np.sign(xb))
        bad = ~ok
    elif dtype == O.F32:
        bad = np.abs(got_deq - x) > eps + ax * 2.0 ** -24
    else:
        raise ValueError(dtype)
    assert not bad.any(), "%d values are not a correct rounding (first at %s)" % (bad.sum(), np.argwhere(bad)[:3])
    if got_codes is not None and dtype != O.F32:
        same = np.mean(got_codes == want_codes)
        assert same >= 0.999, "only %.5f of the codes match" % same


def check_logits(got, want, bound_scale, rows_n):
    for r, n in enumerate(rows_n):
        d = np.abs(got[r, :n].astype(np.float64) - want[r, :n])
        tol = 2e-5 * bound_scale[r, :n] + 1e-30
        assert (d <= tol).all(), "row %d: %d logits off (max excess %.3g)" % (r, (d > tol).sum(), (d - tol).max())


def check_topk_band(got_idx, ora_logits, n, k):
    """R-14 style set check for one row."""
    take = min(k, n)
    sel = got_idx[got_idx >= 0]
    assert len(sel) == take, (len(sel), take)
    assert len(np.unique(sel)) == take
    assert sel.min() >= 0 and sel.max() < n
    if n <= k:
        return 0
    l = ora_logits[:n]
    Lk = np.sort(l)[::-1][k - 1]
    tau = 1e-3 * abs(Lk)
    must = np.flatnonzero(l > Lk + tau)
    never = np.flatnonzero(l < Lk - tau)
    s = set(sel.tolist())
    assert all(g in s for g in must), "entries above the band missing"
    assert not any(g in s for g in never), "entries below the band selected"
    ora = set(np.lexsort((np.arange(n), -l))[:k].tolist())
    return len(s ^ ora) // 2


def check_attention(got, want, kind, out_bf16=False, rel_l2=True):
    """out_bf16: the device output is stored in bf16, whose own rounding
    (half an ulp of the value) is added to the tolerance.  rel_l2=False for
    comparisons across two different (both valid) top-k selections: one
    entry swapped inside the tie band moves a flat-softmax output by about
    1/k of a value vector, some 2 % of the output's norm, while max-abs and
    mean-abs stay within their bounds."""
    got = got.astype(np.float64)
    d = np.abs(got - want)
    if out_bf16:
        d = np.maximum(d - 0.5 * ulp_bf16(want), 0.0)
    if kind == "f32":
        assert d.max() <= 1e-5, "max-abs %.3g" % d.max()
        return
    max_abs = 5e-2 if kind == "mxfp4" else 2e-2
    assert d.max() <= max_abs, "max-abs %.3g > %.3g" % (d.max(), max_abs)
    assert d.mean() <= 2e-3, "mean-abs %.3g" % d.mean()
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    assert rel <= 1e-2 or not rel_l2, "relative L2 %.3g" % rel
