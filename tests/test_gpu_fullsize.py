"""Parity at the full workload sizes, in the launch configuration the
benchmark times (its `Workload`, one step on the device), against the oracle
on sampled query rows:

* compress_append: every entry the step writes is a correct rounding of the
  group's exact aggregate (recomputed here from the group's tokens with the
  oracle's fp64 aggregation), at least 99.9% of its codes equal the oracle's,
  no other pool row changes, and the window and remainder rings are
  bit-exact;
* index_logits within the fp32 summation bound, top-k exact outside the
  tie band (tau = 1e-3 |L_k|);
* attention within max-abs 2e-2 / mean-abs 2e-3 / relative L2 1e-2 (max-abs
  5e-2 for MXFP4 pools) of the oracle, both given the device's selection and
  given the oracle's own, on the raw fp32 outputs the benchmark times; a
  separate case runs the headline step with bf16 outputs, where the output's
  own rounding (half a bf16 ulp of the value, up to 0.0625 at the outlier
  channels' magnitudes) is discounted; log-sum-exp within 2e-3.

`test_prefill_all_rows` checks every one of prefill_8k's 8,192 rows (logits,
top-k band and attention) against the oracle, in chunks of rows.

The initial state is copied to the host before the device step, so the
oracle runs from the same bytes."""
import numpy as np
import pytest
import torch

import bench
import compare as C
import oracle as O
from long_context_compressed_append_amd import lcca, synth
from state import pool_rows

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ODT = {synth.BF16: O.BF16, synth.FP8: O.FP8, synth.MXFP4: O.MXFP4}


def _say(*a):
    print(*a, flush=True)


def _sample(nrows, cap=16):
    if nrows <= cap:
        return np.arange(nrows)
    q = cap // 4
    mid = np.linspace(q, nrows - q - 1, cap - 2 * q).astype(np.int64)
    return np.unique(np.r_[0:q, mid, nrows - q:nrows])


def _run(name, out="f32"):
    _say("full-size parity", name, "building, attention output", out)
    wl = bench.Workload(name, torch, lcca, synth, cold=False, out_dtype=out)
    torch.cuda.synchronize()
    wl.snapshot_host()
    _say(name, "device step")
    wl.step(0)
    torch.cuda.synchronize()
    return wl


class Host:
    """The oracle's copy of the state, after its own compress_append.

    `adopt_device_pools` then replaces the pools and rings with the device's
    (once `_check_compress` has shown every device code to be a correct
    rounding), so the later stages are checked on identical inputs: a code
    may legitimately differ from the oracle's by one rounding step (at most
    0.1 % of them), and a logit scored from the other code differs by more
    than the fp32 summation bound.  The end-to-end check keeps the oracle's
    own state (`own`)."""

    def __init__(self, wl):
        h, c = wl.host, wl.cfg
        self.h, self.c = h, c
        self.bt = np.ascontiguousarray(h["block_table"])
        self.kv = {"dtype": ODT[c.kv_dtype], "data": h["kv_data"].copy(),
                   "scale": h["kv_scale"].copy() if h["kv_scale"] is not None else None}
        self.ik = {"dtype": ODT[c.ik_dtype], "data": h["ik_data"].copy(), "scale": None} if c.HI else None
        self.win = {"dtype": ODT[c.win_dtype], "cap": c.win_cap, "data": h["win_data"].copy(),
                    "scale": h["win_scale"].copy() if h["win_scale"] is not None else None}
        self.rem = {"kv": h["rem_kv"].copy(), "ik": h["rem_ik"].copy() if c.HI else None,
                    "kv_logit": h["rem_kv_logit"].copy(), "ik_logit": h["rem_ik_logit"].copy() if c.HI else None}
        O.compress_append(self.bt, h["cu_new"], h["start_pos"], O.BF16, h["new_kv"].view(np.uint16),
                          h["new_kv_logit"], h["new_ik"].view(np.uint16) if c.HI else None,
                          h["new_ik_logit"] if c.HI else None, c.m, c.D, c.dI, self.kv, self.ik, self.win, self.rem)

    def adopt_device_pools(self, wl):
        kv, ik, win, rem = wl.copies[0]
        self.own = {"kv": self.kv, "ik": self.ik, "win": self.win}
        self.kv = dict(self.kv, data=kv.data.cpu().numpy(),
                       scale=kv.scale.cpu().numpy() if kv.scale is not None else None)
        if ik is not None:
            self.ik = dict(self.ik, data=ik.data.cpu().numpy())
        self.win = dict(self.win, data=win.data.cpu().numpy(),
                        scale=win.scale.cpu().numpy() if win.scale is not None else None)

    def group(self, stream, b, g):
        """Token values (float64 [m][dim]) and logits of group g of sequence b,
        from the initial remainder ring and the step's new tokens."""
        h, c = self.h, self.c
        dim = c.D if stream == "kv" else c.dI
        ring = O.bf16_decode(h["rem_" + stream].view(np.uint16)).reshape(c.batch, c.m, dim)
        ring_a = h["rem_%s_logit" % stream].reshape(c.batch, c.m)
        new = h["new_" + stream].view(np.uint16).reshape(-1, dim)
        new_a = h["new_%s_logit" % stream]
        P, base = c.prior_len[b], int(h["cu_new"][b])
        x, a = np.empty((c.m, dim)), np.empty(c.m)
        for i, p in enumerate(range(g * c.m, (g + 1) * c.m)):
            if p < P:
                x[i], a[i] = ring[b, p % c.m], ring_a[b, p % c.m]
            else:
                x[i], a[i] = O.bf16_decode(new[base + p - P]), new_a[base + p - P]
        return x, a

    def seq_keys(self, store, dim, b, n):
        """Dequantised entries 0..n-1 of sequence b (float64 [n][dim])."""
        E = 256 // self.c.m
        out = np.empty((n, dim))
        for j in range(0, n, E):
            cnt = min(E, n - j)
            out[j:j + cnt] = O.load_rows(store["dtype"], store["data"], store["scale"], int(self.bt[b, j // E]) * E,
                                         cnt, dim)
        return out


def _check_compress(wl, ho):
    c = wl.cfg
    kv, ik, win, rem = wl.copies[0]
    for stream, dev, ora, init, dim in (("kv", kv, ho.kv, "kv", c.D), ("ik", ik, ho.ik, "ik", c.dI)):
        if dev is None:
            continue
        rb = O.row_bytes(ora["dtype"], dim)
        gdata = dev.data.cpu().numpy()
        nrow = gdata.size // rb
        groups, rows = [], []
        for b in range(c.batch):
            for g in range(c.prior_len[b] // c.m, c.total_len(b) // c.m):
                groups.append((b, g))
                rows.append(int(pool_rows(ho.bt, c.m, b, [g])[0]))
        rows = np.asarray(rows, np.int64)
        other = np.ones(nrow, bool)
        other[rows] = False
        assert np.array_equal(gdata.reshape(nrow, rb)[other], ho.h[init + "_data"].reshape(nrow, rb)[other]), \
            stream + ": rows outside the completed groups changed"
        exact = np.empty((len(rows), dim))
        eps = np.empty((len(rows), dim))
        for i, (b, g) in enumerate(groups):
            x, a = ho.group(stream, b, g)
            exact[i] = O.group_compress(x, a)
            eps[i] = (c.m + 8) * 2.0 ** -24 * O.group_compress(np.abs(x), a)
        gscale = dev.scale.cpu().numpy() if dev.scale is not None else None
        got = np.stack([O.load_rows(ora["dtype"], gdata, gscale, int(r), 1, dim)[0] for r in rows])
        gsc = gscale.reshape(nrow, -1)[rows] if ora["dtype"] == O.MXFP4 else None
        C.check_correct_rounding(ora["dtype"], got, exact.astype(np.float32), eps, gdata.reshape(nrow, rb)[rows],
                                 ora["data"].reshape(nrow, rb)[rows], dim, gsc)
        _say(wl.name, stream, "entries written:", len(rows))
    assert np.array_equal(win.data.cpu().numpy(), ho.win["data"])
    if ho.win["scale"] is not None:
        assert np.array_equal(win.scale.cpu().numpy(), ho.win["scale"])
    assert np.array_equal(rem.kv.cpu().numpy(), ho.rem["kv"])
    assert np.array_equal(rem.kv_logit.cpu().numpy(), ho.rem["kv_logit"])
    if c.HI:
        assert np.array_equal(rem.ik.cpu().numpy(), ho.rem["ik"])
        assert np.array_equal(rem.ik_logit.cpu().numpy(), ho.rem["ik_logit"])


def _kind(c):
    return "mxfp4" if c.kv_dtype == synth.MXFP4 else "bf16"


@pytest.mark.parametrize("name,out", [("csa_64k", "f32"), ("csa_64k", "bf16"), ("hca_1m", "f32"),
                                      ("lp_512k", "f32"), ("prefill_8k", "f32")])
def test_full_size_step(name, out):
    wl = _run(name, out)
    c, h = wl.cfg, wl.host
    ho = Host(wl)
    _say(name, "compress_append")
    _check_compress(wl, ho)
    ho.adopt_device_pools(wl)
    rows = _sample(wl.nrows)
    rs, rp = h["row_seq"][rows], h["row_pos"][rows]
    n_r = (rp.astype(np.int64) + 1) // c.m
    q = h["q"].view(np.uint16).reshape(wl.nrows, c.H, c.D)[rows]
    idx = None
    if c.HI:
        _say(name, "index_logits / topk_select on rows", rows.tolist())
        qi = h["q_idx"].view(np.uint16).reshape(wl.nrows, c.HI, c.dI)[rows]
        w = h["w_idx"][rows]
        ol = O.index_logits(rs, rp, c.m, ho.bt, O.BF16, qi, c.HI, c.dI, w, 1.0, ho.ik, wl.ld)
        keys, bound = {}, np.zeros((len(rows), wl.ld))
        qf = np.abs(O.bf16_decode(qi).astype(np.float64))
        for i in range(len(rows)):
            b = int(rs[i])
            if b not in keys:
                keys[b] = np.abs(ho.seq_keys(ho.ik, c.dI, b, int(n_r[rs == b].max())))
            n = int(n_r[i])
            bound[i, :n] = (w[i][:, None] * (qf[i] @ keys[b][:n].T)).sum(0)
        del keys
        lg = wl.logits[torch.from_numpy(rows).cuda()].cpu().numpy()
        C.check_logits(lg, ol, bound, n_r)
        idx = wl.topk[torch.from_numpy(rows).cuda()].cpu().numpy()
        swaps = sum(C.check_topk_band(idx[i], ol[i], int(n_r[i]), c.k) for i in range(len(rows)))
        _say(name, "top-k swaps inside the tie band:", swaps)
    else:
        swaps = 0
    _say(name, "sparse_attn_fwd")
    out = wl.out[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    lse = wl.lse[torch.from_numpy(rows).cuda()].cpu().numpy()
    o_sel, l_sel = O.sparse_attn(rs, rp, c.m, ho.bt, O.BF16, q, c.H, c.D, c.dv, c.scale, ho.kv, idx,
                                 c.k if c.HI else 0, ho.win, c.window)
    C.check_attention(out, o_sel, _kind(c), out_bf16=wl.out_dtype == "bf16")
    assert np.abs(lse - l_sel).max() <= 2e-3
    # end to end: the oracle's own pools, logits and selection
    idx_own = None
    if c.HI:
        ol_own = O.index_logits(rs, rp, c.m, ho.bt, O.BF16, qi, c.HI, c.dI, w, 1.0, ho.own["ik"], wl.ld)
        idx_own = O.topk(rp, c.m, ol_own, c.k)
    o_ora, _ = O.sparse_attn(rs, rp, c.m, ho.bt, O.BF16, q, c.H, c.D, c.dv, c.scale, ho.own["kv"], idx_own,
                             c.k if c.HI else 0, ho.own["win"], c.window)
    # (the two selections may differ inside the tie band: max-abs and mean-abs only then)
    same = idx_own is None or all(set(idx[i].tolist()) == set(idx_own[i].tolist()) for i in range(len(rows)))
    C.check_attention(out, o_ora, _kind(c), out_bf16=wl.out_dtype == "bf16", rel_l2=same)
    _say(name, "ok: max-abs %.3g" % np.abs(out - o_sel).max())


@pytest.mark.timeout(1500)
def test_prefill_all_rows():
    """Every row of the prefill_8k chunk: logits within the fp32 bound, top-k
    exact outside the tie band, attention (raw fp32 outputs) within the bounds
    given the device's selection, and given the oracle's own selection for
    the rows where the two differ inside the band."""
    name = "prefill_8k"
    wl = _run(name)
    c, h = wl.cfg, wl.host
    ho = Host(wl)
    _check_compress(wl, ho)
    ho.adopt_device_pools(wl)
    nr = wl.nrows
    assert nr == 8192
    keys = np.abs(ho.seq_keys(ho.ik, c.dI, 0, c.max_entries))
    qi_all = h["q_idx"].view(np.uint16).reshape(nr, c.HI, c.dI)
    q_all = h["q"].view(np.uint16).reshape(nr, c.H, c.D)
    worst, swaps, checked = 0.0, 0, 0
    chunk = 512
    for r0 in range(0, nr, chunk):
        rows = np.arange(r0, min(nr, r0 + chunk))
        rs, rp = h["row_seq"][rows], h["row_pos"][rows]
        n_r = (rp.astype(np.int64) + 1) // c.m
        qi, w = qi_all[rows], h["w_idx"][rows]
        ol = O.index_logits(rs, rp, c.m, ho.bt, O.BF16, qi, c.HI, c.dI, w, 1.0, ho.ik, wl.ld)
        qf = np.abs(O.bf16_decode(qi).astype(np.float64))
        bound = np.zeros((len(rows), wl.ld))
        for i in range(len(rows)):
            n = int(n_r[i])
            bound[i, :n] = (w[i][:, None] * (qf[i] @ keys[:n].T)).sum(0)
        sel = torch.from_numpy(rows).cuda()
        C.check_logits(wl.logits[sel].cpu().numpy(), ol, bound, n_r)
        idx = wl.topk[sel].cpu().numpy()
        oi = O.topk(rp, c.m, ol, c.k)
        diff = []
        for i in range(len(rows)):
            s_ = C.check_topk_band(idx[i], ol[i], int(n_r[i]), c.k)
            swaps += s_
            if s_:
                diff.append(i)
        q = q_all[rows]
        out = wl.out[sel].float().cpu().numpy()
        lse = wl.lse[sel].cpu().numpy()
        o_sel, l_sel = O.sparse_attn(rs, rp, c.m, ho.bt, O.BF16, q, c.H, c.D, c.dv, c.scale, ho.kv, idx, c.k,
                                     ho.win, c.window)
        C.check_attention(out, o_sel, _kind(c))
        assert np.abs(lse - l_sel).max() <= 2e-3
        if diff:
            d = np.asarray(diff)
            o_ora, _ = O.sparse_attn(rs[d], rp[d], c.m, ho.bt, O.BF16, q[d], c.H, c.D, c.dv, c.scale, ho.kv, oi[d],
                                     c.k, ho.win, c.window)
            C.check_attention(out[d], o_ora, _kind(c), rel_l2=False)
        worst = max(worst, float(np.abs(out - o_sel).max()))
        checked += len(rows)
        _say(name, "rows %d..%d ok (max-abs so far %.3g, top-k swaps inside the band %d)"
             % (rows[0], rows[-1], worst, swaps))
    assert checked == nr
