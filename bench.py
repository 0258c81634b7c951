#!/usr/bin/env python3
"""Decode and chunked-prefill benchmark of compressed-KV attention on one MI355X.

One step is the whole hot path for one batch of query rows:
compress_append -> index_logits -> topk_select -> sparse_attn_fwd (+ the
split merge), all launched back to back on one HIP stream through liblcca's
C ABI.  Inputs are seeded synthetic tensors generated on the device with
torch (N(0,1) values, 1% outlier channels x8 where the workload has them,
caches encoded by torch casts: bf16 RNE, FP8 E4M3 RNE with a per-token
scale for windows, raw E4M3 for FP8 indexer keys, OCP MXFP4 with RNE) and
resident in HBM before the timed region starts.

Workloads (one attention layer each):
  csa_64k     16 sequences x 65,536 tokens, m=4 (16,384 bf16 entries each),
              64 query heads, dim 576, indexer 64 x 128, top-k 2,048,
              128-token FP8 window.  This is the line's `value`.
  hca_1m      4 sequences x 1,048,576 tokens, m=128 (8,192 entries each),
              dense attention over every entry plus the window.
  lp_512k     32 sequences x 524,288 tokens, m=4, MXFP4 entries, FP8 indexer
              keys, FP8 window, top-k 2,048.
  prefill_8k  1 sequence: 122,880 prior tokens + an 8,192-token chunk
              compressed and appended; one query row per new token; bf16
              window.

Cold-cache rule: the caches are replicated R times so that R copies exceed
1 GiB (four times the 256 MiB Infinity Cache) and step i reads copy i % R;
`hot` numbers (R = 1) are reported beside.

Per-stage times come from HIP events recorded between the launches on the
stream they run on.  Algorithmic bytes count the unique bytes each stage must
move (`Workload.stage_work`).  The CPU baseline is the oracle (plain fp64 C,
OpenMP over rows) timed on the host on a sample of the headline step, on the
same bytes copied to the host before the first device step; every workload's
sampled rows are also compared with the oracle (`parity`).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads a,b]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode query-rows/s + achieved HBM GB/s (% peak) at 64K/1M ctx, 1 MI355X"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COLD_BYTES = 1 << 30
CHUNK_ELEMS = 1 << 25                   # device temporaries while encoding large pools


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# device-side encoders (input construction only; the oracle checks them)
# --------------------------------------------------------------------------

def enc_bf16(torch, x):
    return x.to(torch.bfloat16).contiguous().view(torch.uint8).reshape(-1)


def enc_fp8_scaled(torch, x):
    """Per-row scale s = amax/448 (1 for a zero row), codes = RNE(x/s) in E4M3."""
    amax = x.abs().amax(-1, keepdim=True)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (x / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return codes.contiguous().view(torch.uint8).reshape(-1), s.reshape(-1).contiguous()


def enc_fp8_raw(torch, x):
    return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).contiguous().view(torch.uint8).reshape(-1)


def enc_mxfp4(torch, x):
    """OCP MX: per 32 elements X = floor(log2 amax) - 2 (amax 0 -> -127), E2M1
    codes of x / 2^X rounded to nearest even, saturating at 6; element 2i in
    the low nibble.  Returns (codes uint8 [rows*dim/2], scales uint8 [rows*dim/32])."""
    rows, dim = x.shape
    xb = x.reshape(rows, dim // 32, 32)
    amax = xb.abs().amax(-1)
    _, e = torch.frexp(amax)
    X = torch.where(amax > 0, e - 3, torch.full_like(e, -127)).clamp(-127, 127)
    a = torch.ldexp(xb.abs(), -X.unsqueeze(-1).to(torch.float32))
    code = ((a > 0.25).int() + (a >= 0.75).int() + (a > 1.25).int() + (a >= 1.75).int() + (a > 2.5).int()
            + (a >= 3.5).int() + (a > 5.0).int())
    nib = (code | (torch.signbit(xb).int() << 3)).reshape(rows, dim // 2, 2)
    data = (nib[..., 0] | (nib[..., 1] << 4)).to(torch.uint8).reshape(-1)
    scale = (X + 127).to(torch.uint8).reshape(-1)
    return data, scale


# --------------------------------------------------------------------------
# workload construction (device-side, seeded)
# --------------------------------------------------------------------------

def stage_work(c, gated=False):
    """Algorithmic (bytes, flops) per stage: the unique bytes each stage
    must read and write (every cache row counted once per step, however
    many rows or heads use it) and the multiply-adds it must do.  gated:
    compress_append with a logit per token and channel."""
    import numpy as np
    m, D, H, HI, dI, k, w = c.m, c.D, c.H, c.HI, c.dI, c.k, c.window
    kv_row = {"bf16": 2 * D, "mxfp4": D // 2 + D // 32}[c.kv_dtype]
    ik_row = {"bf16": 2 * dI, "fp8": dI}[c.ik_dtype] if HI else 0
    win_row = {"fp8": D + 4, "bf16": 2 * D}[c.win_dtype]
    if gated:                                               # bf16 token + its logit row, both streams
        tok_row = 6 * D + (6 * dI if HI else 0)
    else:                                                   # bf16 token + its logit, both streams
        tok_row = 2 * D + 4 + ((2 * dI + 4) if HI else 0)
    seq, pos = c.rows_of()
    pos = pos.astype(np.int64)
    n_r = (pos + 1) // m
    nwin = np.minimum(pos + 1, w)
    nsel = np.minimum(n_r, k) if HI else n_r
    comp = idx_b = topk_b = attn_b = 0
    for b in range(c.batch):
        P, T, nn = c.prior_len[b], c.total_len(b), c.n_new[b]
        groups = T // m - P // m
        ring_in = (P % m) if groups else 0                  # earlier tokens of the first completed group
        tail = min(nn, T % m)                               # new tokens left in the remainder ring
        comp += nn * (tok_row + win_row) + ring_in * tok_row + tail * tok_row + groups * (kv_row + ik_row)
        sel = seq == b
        if not sel.any():
            continue
        nb = c.blocks_per_seq(b)
        keys = int(n_r[sel].max())                          # every visible key of the sequence, once
        if HI:
            idx_b += keys * ik_row + nb * 4 + int(sel.sum()) * (HI * dI * 2 + 4 * HI) + 4 * int(n_r[sel].sum())
            topk_b += 4 * int(n_r[sel].sum()) + 4 * k * int(sel.sum())
        span = int(pos[sel].max() - max(0, pos[sel].min() - w + 1) + 1)
        attn_b += (min(int(nsel[sel].sum()), keys) * kv_row + (4 * k * int(sel.sum()) if HI else 0)
                   + min(int(nwin[sel].sum()), span) * win_row)
    nrows = len(pos)
    attn_b += nrows * (H * D * 2 + H * c.dv * 2 + 4 * H)
    idx_f = int(2 * HI * dI * n_r.sum()) if HI else 0
    attn_f = int(2 * H * (D + c.dv) * (nsel + nwin).sum())
    return {"compress_append": (int(comp), 0), "index_logits": (int(idx_b), idx_f),
            "topk_select": (int(topk_b), 0), "sparse_attn_fwd": (int(attn_b), attn_f)}


class Workload:
    """Device tensors of one step of a workload and R rotated cache copies."""

    def __init__(self, name, torch, lcca, synth, cold=True, out_dtype="f32"):
        self.name = name
        self.cfg = c = synth.CONFIGS[name]
        self.torch, self.lcca = torch, lcca
        dev = "cuda"
        B, m, D, H, HI, dI = c.batch, c.m, c.D, c.H, c.HI, c.dI
        self.B = B
        E = c.E
        nb = c.max_blocks
        nblk = c.num_blocks
        self.seed_base = (0x1CCA << 16) | (c.cfg_id << 8)
        assert c.tok_dtype == synth.BF16 and c.q_dtype == synth.BF16

        def gen(tid):
            g = torch.Generator(device=dev)
            g.manual_seed(self.seed_base + tid)
            return g

        def outliers(dim, stream):
            n = int(round(c.outlier_frac * dim))
            if n == 0 or dim == 0:
                return None
            g = torch.Generator()
            g.manual_seed(self.seed_base + 100 + stream)
            return torch.randperm(dim, generator=g)[:n].to(dev)

        och = {0: outliers(D, 0), 1: outliers(dI, 1)}

        def values(g, shape, stream):
            x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
            ch = och[stream]
            if ch is not None:
                x[..., ch] *= c.outlier_mult
            return x

        def rows_of(tid, nrows, dim, stream, enc):
            """nrows x dim values of one stream, encoded chunk by chunk."""
            g = gen(tid)
            step = max(1, CHUNK_ELEMS // dim)
            parts, scales = [], []
            for r0 in range(0, nrows, step):
                x = values(g, (min(step, nrows - r0), dim), stream)
                out = enc(x)
                if isinstance(out, tuple):
                    parts.append(out[0]); scales.append(out[1])
                else:
                    parts.append(out)
                del x
            data = torch.cat(parts) if len(parts) > 1 else parts[0]
            sc = (torch.cat(scales) if len(scales) > 1 else scales[0]) if scales else None
            return data, sc

        bf16 = lambda x: enc_bf16(torch, x)
        kv_enc = {synth.BF16: bf16, synth.MXFP4: lambda x: enc_mxfp4(torch, x)}[c.kv_dtype]
        ik_enc = {synth.BF16: bf16, synth.FP8: lambda x: enc_fp8_raw(torch, x)}[c.ik_dtype] if HI else None
        win_enc = {synth.FP8: lambda x: enc_fp8_scaled(torch, x), synth.BF16: bf16}[c.win_dtype]
        LDT = {synth.BF16: lcca.BF16, synth.FP8: lcca.FP8_E4M3, synth.MXFP4: lcca.MXFP4}
        self.kv_dt, self.win_dt = LDT[c.kv_dtype], LDT[c.win_dtype]
        self.ik_dt = LDT[c.ik_dtype] if HI else None

        g = torch.Generator()
        g.manual_seed(self.seed_base + 15)
        perm = torch.randperm(nblk, generator=g).to(torch.int32)
        bt = torch.zeros((B, nb), dtype=torch.int32)
        o = 0
        for b in range(B):
            k = c.blocks_per_seq(b)
            bt[b, :k] = perm[o:o + k]
            o += k
        self.block_table = bt.contiguous().to(dev)

        kv_data, kv_scale = rows_of(1, nblk * E, D, 0, kv_enc)
        ik_data = rows_of(2, nblk * E, dI, 1, ik_enc)[0] if HI else None
        win_data, win_scale = rows_of(3, B * c.win_cap, D, 0, win_enc)
        rem_kv = rows_of(4, B * m, D, 0, bf16)[0]
        rem_ik = rows_of(5, B * m, dI, 1, bf16)[0] if HI else None
        rem_kv_logit = torch.randn(B * m, generator=gen(6), device=dev)
        rem_ik_logit = torch.randn(B * m, generator=gen(7), device=dev) if HI else None
        total_new = sum(c.n_new)
        self.total_new = total_new
        self.new_kv = rows_of(8, total_new, D, 0, bf16)[0]
        self.new_ik = rows_of(9, total_new, dI, 1, bf16)[0] if HI else None
        self.new_kv_logit = torch.randn(total_new, generator=gen(10), device=dev)
        self.new_ik_logit = torch.randn(total_new, generator=gen(11), device=dev) if HI else None

        rs, rp = c.rows_of()
        self.nrows = len(rs)
        self.row_seq = torch.from_numpy(rs).to(dev)
        self.row_pos = torch.from_numpy(rp).to(dev)
        self.row_pos_host = rp
        self.max_pos = int(rp.max())
        self.q = rows_of(12, self.nrows * H, D, 0, bf16)[0]
        self.q_idx = rows_of(13, self.nrows * HI, dI, 1, bf16)[0] if HI else None
        self.w_idx = torch.rand((self.nrows, HI), generator=gen(14), device=dev) if HI else None

        self.cu_new = torch.tensor([0] + list(torch.tensor(c.n_new).cumsum(0).tolist()), dtype=torch.int32,
                                   device=dev)
        self.start_pos = torch.tensor(list(c.prior_len), dtype=torch.int32, device=dev)
        self.ld = c.max_entries
        self.pages = lcca.Pages(self.block_table)
        self.rows = lcca.Rows(self.row_seq, self.row_pos, self.max_pos)

        self.host = None
        self.q_ldt = lcca.BF16          # indexer query dtype (| lcca.Q_FP8: FP8 queries)
        self.a_qdt = lcca.BF16          # attention query dtype (| lcca.Q_FP8 on MXFP4 pools)
        self._init = dict(kv_data=kv_data, kv_scale=kv_scale, ik_data=ik_data, win_data=win_data,
                          win_scale=win_scale, rem_kv=rem_kv, rem_ik=rem_ik, rem_kv_logit=rem_kv_logit,
                          rem_ik_logit=rem_ik_logit)
        self.footprint = sum(t.numel() * t.element_size() for t in self._init.values() if t is not None)
        self.R = max(1, math.ceil(COLD_BYTES / self.footprint)) if cold else 1
        self.copies = []
        for i in range(self.R):
            t = self._init if i == 0 else {k: (v.clone() if v is not None else None) for k, v in self._init.items()}
            kv = lcca.PagedCache(self.kv_dt, D, m, nblk, t["kv_data"], t["kv_scale"])
            ik = lcca.PagedCache(self.ik_dt, dI, m, nblk, t["ik_data"]) if HI else None
            win = lcca.WindowCache(self.win_dt, D, c.win_cap, c.window, t["win_data"], t["win_scale"])
            rem = lcca.Remainder(lcca.BF16, t["rem_kv"], t["rem_kv_logit"], t["rem_ik"], t["rem_ik_logit"])
            self.copies.append((kv, ik, win, rem))
        self.logits = torch.empty((self.nrows, max(self.ld, 1)), dtype=torch.float32, device=dev) if HI else None
        self.topk = torch.empty((self.nrows, max(c.k, 1)), dtype=torch.int32, device=dev) if HI else None
        self.set_out_dtype(out_dtype)
        self.lse = torch.empty((self.nrows, H), dtype=torch.float32, device=dev)
        wsb = lcca.sparse_attn_workspace_size(self.rows, m, H, D, c.dv, c.k, bool(HI), c.window)
        self.ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
        tkb = lcca.topk_workspace_size(self.rows, m, c.k) if HI else 0
        self.topk_ws = torch.empty(tkb, dtype=torch.uint8, device=dev) if tkb else None
        # decode steps with one new token and one row per sequence run
        # compress_append, index_logits and topk_select as lcca_decode_select
        # (one launch fewer) when its selection covers the rows: up to 32K
        # entries, or 16K-entry slices whose top-k candidates total <= 32K
        slices = 1 if self.ld <= 32768 else -(-self.ld // 16384)
        self.fused = bool(HI) and c.rows == "last" and all(n == 1 for n in c.n_new) and self.ld % 4 == 0 \
            and (slices == 1 or slices * c.k <= 32768)
        # its workspace: allocated zeroed once, left zeroed by every call
        self.ds_ws = torch.zeros(max(lcca.decode_select_workspace_size(self.rows, m, c.k), 16), dtype=torch.uint8,
                                 device=dev) if self.fused else None

    def set_out_dtype(self, out_dtype):
        """Attention output in fp32 ("f32") or bf16 ("bf16")."""
        torch, c = self.torch, self.cfg
        self.out_dtype = out_dtype
        self.out_ldt = self.lcca.F32 if out_dtype == "f32" else self.lcca.BF16
        self.out = torch.empty((self.nrows, c.H, c.dv), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16,
                               device="cuda")

    def snapshot_host(self):
        """Copy the initial state to host numpy arrays (for the oracle)."""
        h = {k: (v.cpu().numpy() if v is not None else None) for k, v in self._init.items()}
        for k in ("new_kv", "new_ik", "new_kv_logit", "new_ik_logit", "q", "q_idx", "w_idx", "block_table",
                  "cu_new", "start_pos", "row_seq", "row_pos"):
            v = getattr(self, k)
            h[k] = v.cpu().numpy() if v is not None else None
        self.host = h

    # one step on copy i; `ev` (optional) gets an event after each stage
    def step(self, i, ev=None):
        c, L = self.cfg, self.lcca
        kv, ik, win, rem = self.copies[i % self.R]
        if ev is not None:
            ev[0].record()
        if self.fused:
            L.decode_select(self.pages, self.rows, self.cu_new, self.start_pos, self.total_new, L.BF16, self.new_kv,
                            self.new_kv_logit, self.new_ik, self.new_ik_logit, kv, ik, win, rem, self.q_ldt, self.q_idx,
                            c.HI, self.w_idx, 1.0, self.logits, self.ld, c.k, self.topk, self.ds_ws)
            if ev is not None:
                ev[1].record()
            L.sparse_attn_fwd(self.pages, self.rows, self.a_qdt, self.q, c.H, c.dv, c.scale, kv, self.topk, c.k, win,
                              self.out_ldt, self.out, self.lse, self.ws)
            if ev is not None:
                ev[4].record()
            return
        L.compress_append(self.pages, self.cu_new, self.start_pos, self.total_new, L.BF16, self.new_kv,
                          self.new_kv_logit, self.new_ik, self.new_ik_logit, kv, ik, win, rem)
        if ev is not None:
            ev[1].record()
        idx = None
        if c.HI:
            L.index_logits(self.pages, self.rows, self.q_ldt, self.q_idx, c.HI, self.w_idx, 1.0, ik, self.logits,
                           self.ld)
            if ev is not None:
                ev[2].record()
            L.topk_select(self.rows, c.m, self.logits, self.ld, c.k, self.topk, self.topk_ws)
            idx = self.topk
        elif ev is not None:
            ev[2].record()
        if ev is not None:
            ev[3].record()
        L.sparse_attn_fwd(self.pages, self.rows, self.a_qdt, self.q, c.H, c.dv, c.scale, kv, idx,
                          c.k if idx is not None else 0, win, self.out_ldt, self.out, self.lse, self.ws)
        if ev is not None:
            ev[4].record()

def time_steps(torch, wl, steps, warmup):
    """Mean step time and per-stage mean times (ms) over `steps` timed steps."""
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        wl.step(i, evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3 / steps
    total = t0.elapsed_time(t1) / steps
    if wl.fused:
        names, pairs = ("decode_select", "sparse_attn_fwd"), ((0, 1), (1, 4))
    else:
        names = ("compress_append", "index_logits", "topk_select", "sparse_attn_fwd")
        pairs = ((0, 1), (1, 2), (2, 3), (3, 4))
    stage = {}
    for n, (a, b) in zip(names, pairs):
        stage[n] = sum(e[a].elapsed_time(e[b]) for e in evs) / steps
    return total, stage, wall


def plain_steps(torch, wl, steps):
    """Step time with no events between the stages (ms)."""
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        wl.step(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


# --------------------------------------------------------------------------
# the oracle on sampled rows of the same step
# --------------------------------------------------------------------------

def sample_rows(wl, max_rows=16):
    n = wl.nrows
    if n <= max_rows:
        return list(range(n))
    half = max_rows // 2
    return list(range(half)) + list(range(n - half, n))


def oracle_rows(wl, rows, min_seconds=0.0):
    """Oracle outputs (out [rows][H][dv] fp64, top-k [rows][k] or None) for the
    given row indices, from the host snapshot.  The pass (compress_append of
    the step, then the three row stages) is repeated until min_seconds of wall
    time are spent; compress_append is idempotent at fixed positions, so every
    pass computes the same.  Returns the outputs, the logits, the mean wall
    time of one pass and the number of passes."""
    import numpy as np
    import oracle as O
    h, c = wl.host, wl.cfg
    m, D, dI = c.m, c.D, c.dI
    ODT = {"bf16": O.BF16, "fp8": O.FP8, "mxfp4": O.MXFP4}
    kv = {"dtype": ODT[c.kv_dtype], "data": h["kv_data"].copy(),
          "scale": h["kv_scale"].copy() if h["kv_scale"] is not None else None}
    ik = {"dtype": ODT[c.ik_dtype], "data": h["ik_data"].copy(), "scale": None} if c.HI else None
    win = {"dtype": ODT[c.win_dtype], "cap": c.win_cap, "data": h["win_data"].copy(),
           "scale": h["win_scale"].copy() if h["win_scale"] is not None else None}
    rem = {"kv": h["rem_kv"].copy(), "ik": h["rem_ik"].copy() if c.HI else None,
           "kv_logit": h["rem_kv_logit"].copy(), "ik_logit": h["rem_ik_logit"].copy() if c.HI else None}
    bt = np.ascontiguousarray(h["block_table"])
    rows = np.asarray(rows)
    rs, rp = h["row_seq"][rows], h["row_pos"][rows]
    q = h["q"].view(np.uint16).reshape(wl.nrows, c.H, D)[rows]
    qi = h["q_idx"].view(np.uint16).reshape(wl.nrows, c.HI, dI)[rows] if c.HI else None
    spent, passes = 0.0, 0
    while True:
        t0 = time.perf_counter()
        O.compress_append(bt, h["cu_new"], h["start_pos"], O.BF16, h["new_kv"].view(np.uint16),
                          h["new_kv_logit"], h["new_ik"].view(np.uint16) if c.HI else None,
                          h["new_ik_logit"] if c.HI else None, m, D, dI, kv, ik, win, rem)
        idx = lg = None
        if c.HI:
            lg = O.index_logits(rs, rp, m, bt, O.BF16, qi, c.HI, dI, h["w_idx"][rows], 1.0, ik, wl.ld)
            idx = O.topk(rp, m, lg, c.k)
        out, lse = O.sparse_attn(rs, rp, m, bt, O.BF16, q, c.H, D, c.dv, c.scale, kv, idx, c.k if c.HI else 0,
                                 win, c.window)
        spent += time.perf_counter() - t0
        passes += 1
        if spent >= min_seconds:
            return out, idx, lg, spent / passes, passes


def cpu_baseline(wl, rows, dt, passes):
    import oracle as O
    return {"value": len(rows) / dt, "unit": "query-rows/s", "cores": min(O.num_threads(), len(rows)),
            "kind": "oracle",
            "sample": "%d of %d rows of %s (compress_append of the whole step + index_logits + topk_select + "
                      "sparse_attn for the sampled rows, fp64, OpenMP over rows), %d passes, %.2f s wall each, "
                      "%.1f s in all" % (len(rows), wl.nrows, wl.name, passes, dt, dt * passes)}


def cpu_single_thread(wl, rows):
    """The oracle on one thread: one pass over a few sampled rows."""
    import oracle as O
    n0 = O.num_threads()
    O.set_num_threads(1)
    try:
        _, _, _, dt, _ = oracle_rows(wl, rows)
    finally:
        O.set_num_threads(n0)
    return {"value": round(len(rows) / dt, 3), "unit": "query-rows/s", "cores": 1, "kind": "oracle",
            "sample": "%d of %d rows of %s (compress_append of the whole step + the three row stages), one pass, "
                      "%.2f s" % (len(rows), wl.nrows, wl.name, dt)}


# BASELINE bounds for bf16/FP8 paths (MXFP4 pools: max-abs 5e-2)
PARITY_BOUNDS = {"max_abs": 2e-2, "mean_abs": 2e-3, "rel_l2": 1e-2}


def parity_summary(wl, rows, out_ref, idx_ref):
    """Device output against the oracle's fp64 output on the sampled rows, on
    the raw values.  A bf16 output also reports `max_abs_excess`, the error
    beyond its own rounding (half an ulp of the oracle's value)."""
    import numpy as np
    got = wl.out[rows].float().cpu().numpy().astype(np.float64)
    d = np.abs(got - out_ref)
    res = {"rows": len(rows), "out_dtype": wl.out_dtype, "max_abs": float(d.max()), "mean_abs": float(d.mean()),
           "rel_l2": float(np.linalg.norm(got - out_ref) / max(np.linalg.norm(out_ref), 1e-30))}
    if wl.out_dtype == "bf16":
        a = np.abs(out_ref)
        half_ulp = 0.5 * 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))).clip(-126) - 7)
        res["max_abs_excess"] = float(np.maximum(d - half_ulp, 0).max())
    bounds = dict(PARITY_BOUNDS, max_abs=5e-2 if wl.cfg.kv_dtype == "mxfp4" else PARITY_BOUNDS["max_abs"])
    res["bounds"] = bounds
    res["within_bounds"] = bool(all(res[k] <= v for k, v in bounds.items()))
    if idx_ref is not None:
        gi = wl.topk[rows].cpu().numpy()
        res["topk_set_diff"] = int(sum(len(set(gi[i].tolist()) ^ set(idx_ref[i].tolist())) // 2
                                       for i in range(len(rows))))
    return res


# --------------------------------------------------------------------------
# HBM traffic measured by rocprofv3 counters (profiles/), if still current
# --------------------------------------------------------------------------

# the source files of each stage's kernels
STAGE_SOURCES = {"compress_append": ("compress_append.hip", "compress_dev.h"),
                 "index_logits": ("index_logits.hip",),
                 "topk_select": ("topk_select.hip", "compress_dev.h"),
                 "sparse_attn_fwd": ("sparse_attn.hip",),
                 "decode_select": ("index_logits.hip", "topk_select.hip", "compress_dev.h")}


def kernel_source_hash(fnames):
    h = hashlib.sha256()
    for f in fnames:
        h.update(open(os.path.join(ROOT, "long_context_compressed_append_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, stage):
    """Per-step HBM bytes of a stage from profiles/hbm_traffic.txt when the
    line for (workload, stage) carries the current hash of the stage's kernel
    sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    want = kernel_source_hash(STAGE_SOURCES[stage])
    kernel = stage
    for line in open(path):
        f = line.split()
        if len(f) >= 4 and f[0] == workload and f[1] == kernel and f[2] == want:
            return float(f[3])
    return None


def gated_leg(torch, lcca, wl, steps, warmup):
    """Mean time (ms) of lcca_compress_append_gated on the workload's new
    tokens, with N(0,1) logits per token and channel, over the rotated cache
    copies (the same positions each call, so every call stores the same
    bytes)."""
    c = wl.cfg
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed_base + 17)
    nk = torch.randn((wl.total_new, c.D), generator=g, device="cuda")
    ni = torch.randn((wl.total_new, c.dI), generator=g, device="cuda") if c.HI else None
    rk = torch.randn((wl.B * c.m, c.D), generator=g, device="cuda")
    ri = torch.randn((wl.B * c.m, c.dI), generator=g, device="cuda") if c.HI else None
    rems = [lcca.Remainder(lcca.BF16, rem.kv, rk, rem.ik, ri) for (_, _, _, rem) in wl.copies]

    def call(i):
        kv, ik, win, _ = wl.copies[i % wl.R]
        lcca.compress_append_gated(wl.pages, wl.cu_new, wl.start_pos, wl.total_new, lcca.BF16, wl.new_kv, nk,
                                   wl.new_ik, ni, kv, ik, win, rems[i % wl.R])

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        call(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def rope_leg(torch, lcca, wl, steps, warmup):
    """Time the rotary embeddings of one step, each on a copy of its tensor:
    the attention queries and the new tokens (64 RoPE dims at the end of the
    shared vector), the indexer queries and keys (their first 64 dims), and
    the inverse rotation of the attention output's last 64 dims.  Returns
    {call: (ms, bytes)} with bytes = the slice read and written."""
    c = wl.cfg
    pos_rows = wl.row_pos
    pos_tok = torch.cat([torch.arange(p, p + n, dtype=torch.int32, device="cuda")
                         for p, n in zip(c.prior_len, c.n_new)])
    rd = 64
    calls = {"q": (wl.q.clone().view(torch.bfloat16).view(wl.nrows, c.H, c.D), pos_rows, c.D - rd, False),
             "kv_tokens": (wl.new_kv.clone().view(torch.bfloat16).view(wl.total_new, 1, c.D), pos_tok, c.D - rd, False)}
    if c.HI:
        calls["q_idx"] = (wl.q_idx.clone().view(torch.bfloat16).view(wl.nrows, c.HI, c.dI), pos_rows, 0, False)
        calls["ik_tokens"] = (wl.new_ik.clone().view(torch.bfloat16).view(wl.total_new, 1, c.dI), pos_tok, 0, False)
    calls["out_inverse"] = (wl.out.clone(), pos_rows, c.dv - rd, True)
    res = {}
    for name, (x, pos, off, inv) in calls.items():
        for i in range(warmup):
            lcca.rope(x, pos, off, rd, inverse=inv)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            lcca.rope(x, pos, off, rd, inverse=inv)
        t1.record()
        torch.cuda.synchronize()
        b = 2 * x.shape[0] * x.shape[1] * rd * x.element_size()
        res[name] = (t0.elapsed_time(t1) / steps, b)
    return res


def run_workload(torch, lcca, synth, name, args, with_oracle, cpu_seconds=0.0, bf16_variant=False):
    log("workload", name, "building")
    wl = Workload(name, torch, lcca, synth, cold=True, out_dtype="f32")
    torch.cuda.synchronize()
    if with_oracle:
        wl.snapshot_host()
    log("workload", name, "R=%d copies of %.1f MiB, %d rows" % (wl.R, wl.footprint / 2 ** 20, wl.nrows))
    steps = args.steps if wl.nrows <= 1024 else max(1, min(args.steps, args.prefill_steps))
    total, stage, wall = time_steps(torch, wl, steps, args.warmup)
    plain = plain_steps(torch, wl, steps)
    hot_total = None
    if not args.no_hot and wl.R > 1:
        saved = wl.R
        wl.R = 1
        for i in range(args.warmup):
            wl.step(0)
        hot_total = plain_steps(torch, wl, steps)
        wl.R = saved
    work = stage_work(wl.cfg)
    if wl.fused:
        parts = [work.pop(n) for n in ("compress_append", "index_logits", "topk_select")]
        work = {"decode_select": (sum(b for b, _ in parts), sum(f for _, f in parts)), **work}
    step_bytes = sum(b for b, _ in work.values())
    step_flops = sum(f for _, f in work.values())
    per = {}
    for n, (b, f) in work.items():
        t = stage[n]
        if b == 0 and f == 0:
            continue
        e = {"ms": round(t, 5), "GB/s": round(b / t / 1e6, 1) if t > 0 else None,
             "hbm_frac": round(b / t / 1e6 / HBM_PEAK_GBS, 4) if t > 0 else None, "bytes": b}
        if f:
            e["TFLOP/s"] = round(f / t / 1e9, 2)
            e["mfma_frac"] = round(f / t / 1e9 / BF16_PEAK_TFLOPS, 4)
        per[n] = e
    res = {"rows_per_s": wl.nrows / (plain / 1e3), "ms_per_step": plain, "ms_per_step_events": total,
           "wall_ms_per_step": wall, "hot_ms_per_step": hot_total,
           "hot_rows_per_s": wl.nrows / (hot_total / 1e3) if hot_total else None,
           "step_GB/s": step_bytes / plain / 1e6, "step_hbm_frac": step_bytes / plain / 1e6 / HBM_PEAK_GBS,
           "step_TFLOP/s": step_flops / plain / 1e9, "step_bytes": step_bytes, "step_flops": step_flops,
           "stages": per, "R": wl.R, "steps": steps, "rows": wl.nrows}
    baseline = None
    if with_oracle:
        torch.cuda.synchronize()
        rows = sample_rows(wl, args.cpu_sample_rows)
        out_ref, idx_ref, _, dt, passes = oracle_rows(wl, rows, cpu_seconds)
        res["parity"] = parity_summary(wl, rows, out_ref, idx_ref)
        baseline = cpu_baseline(wl, rows, dt, passes)
        res["cpu_1t"] = cpu_single_thread(wl, rows[:4])
        log(name, "oracle %.2f s x %d; parity %s" % (dt, passes, json.dumps(res["parity"])))
    if bf16_variant:
        # the same step with bf16 attention outputs (fp16 split partials)
        wl.set_out_dtype("bf16")
        for i in range(args.warmup):
            wl.step(i)
        t = plain_steps(torch, wl, steps)
        v = {"rows_per_s": round(wl.nrows / (t / 1e3), 1), "ms_per_step": round(t, 5)}
        if with_oracle:
            v["parity"] = parity_summary(wl, rows, out_ref, idx_ref)
        res["bf16_out"] = v
        log(name, "bf16 outputs", json.dumps(v))
    if not args.no_fp8q and wl.cfg.HI and wl.cfg.ik_dtype == synth.FP8 and wl.nrows < 64:
        # the same step with FP8 queries (opt-in): the indexer on the FP8
        # keys, and the attention on an MXFP4 pool by the FP4 x FP8 MFMA
        wl.q_ldt = lcca.BF16 | lcca.Q_FP8
        mx = wl.cfg.kv_dtype == synth.MXFP4
        if mx:
            wl.a_qdt = lcca.BF16 | lcca.Q_FP8
        for i in range(args.warmup):
            wl.step(i)
        t = plain_steps(torch, wl, steps)
        _, st8, _ = time_steps(torch, wl, steps, 0)
        wl.q_ldt = wl.a_qdt = lcca.BF16
        sel = "decode_select" if wl.fused else "index_logits"
        res["fp8_query"] = {"rows_per_s": round(wl.nrows / (t / 1e3), 1), "ms_per_step": round(t, 5)}
        for n in [sel] + (["sparse_attn_fwd"] if mx else []):
            b = work[n][0]
            res["fp8_query"][n] = {"ms": round(st8[n], 5), "GB/s": round(b / st8[n] / 1e6, 1),
                                   "hbm_frac": round(b / st8[n] / 1e6 / HBM_PEAK_GBS, 4)}
        log(name, "fp8 queries", json.dumps(res["fp8_query"]))
    if not args.no_pbf16 and wl.cfg.outlier_frac == 0.0 and wl.cfg.kv_dtype != synth.F32:
        # the same step with the softmax weights as bf16 alone in P.V (opt-in;
        # not on csa_64k, whose 8-sigma outlier channels need the hi + lo pair)
        wl.a_qdt = lcca.BF16 | lcca.P_BF16
        for i in range(args.warmup):
            wl.step(i)
        t = plain_steps(torch, wl, steps)
        _, stp, _ = time_steps(torch, wl, steps, 0)
        b, f = work["sparse_attn_fwd"]
        v = {"rows_per_s": round(wl.nrows / (t / 1e3), 1), "ms_per_step": round(t, 5),
             "sparse_attn_fwd": {"ms": round(stp["sparse_attn_fwd"], 5),
                                 "hbm_frac": round(b / stp["sparse_attn_fwd"] / 1e6 / HBM_PEAK_GBS, 4),
                                 "mfma_frac": round(f / stp["sparse_attn_fwd"] / 1e9 / BF16_PEAK_TFLOPS, 4)}}
        if with_oracle:
            v["parity"] = parity_summary(wl, rows, out_ref, idx_ref)
        wl.a_qdt = lcca.BF16
        res["p_bf16"] = v
        log(name, "bf16 weights", json.dumps(v))
    if not args.no_gated:
        t = gated_leg(torch, lcca, wl, steps, args.warmup)
        b = stage_work(wl.cfg, gated=True)["compress_append"][0]
        res["gated_compress"] = {"ms": round(t, 5), "GB/s": round(b / t / 1e6, 1),
                                 "hbm_frac": round(b / t / 1e6 / HBM_PEAK_GBS, 4), "bytes": b}
        log(name, "compress_append_gated", json.dumps(res["gated_compress"]))
    if not args.no_rope:
        rr = rope_leg(torch, lcca, wl, steps, args.warmup)
        res["rope"] = {k: {"ms": round(t, 5), "GB/s": round(b / t / 1e6, 1), "bytes": b} for k, (t, b) in rr.items()}
        res["rope"]["total_ms"] = round(sum(t for t, _ in rr.values()), 5)
        log(name, "rope", json.dumps(res["rope"]))
    log(name, json.dumps({k: v for k, v in res.items() if k != "stages"}))
    del wl
    torch.cuda.empty_cache()
    return res, baseline


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill-steps", type=int, default=20, help="timed steps of workloads with > 1024 rows")
    ap.add_argument("--workloads", default="csa_64k,hca_1m,lp_512k,prefill_8k")
    ap.add_argument("--no-oracle", action="store_true", help="skip the oracle baseline and parity samples")
    ap.add_argument("--cpu-sample-rows", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the headline workload's oracle pass for at least this long (CPU baseline)")
    ap.add_argument("--no-hot", action="store_true")
    ap.add_argument("--no-fp8q", action="store_true",
                    help="skip the FP8-query indexer leg of workloads with FP8 indexer keys")
    ap.add_argument("--no-rope", action="store_true", help="skip timing the rotary embeddings of a step")
    ap.add_argument("--no-pbf16", action="store_true", help="skip the step with bf16-only softmax weights in P.V")
    ap.add_argument("--no-gated", action="store_true",
                    help="skip the per-channel-gated compress_append leg of each workload")
    ap.add_argument("--no-bf16-variant", action="store_true",
                    help="skip the headline step with bf16 attention outputs (reported beside the fp32 one)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run 10 device copies of BYTES bytes (a reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the decode path is measured on one MI355X "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_compressed_append_amd import lcca, synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 10
        print(json.dumps({"copy_bytes": args.copy_probe, "ms": dt * 1e3, "GB/s": 2 * args.copy_probe / dt / 1e9}))
        return
    lcca.lib()                                    # raises if liblcca.so is missing
    log("lcca", lcca.version(), "device", torch.cuda.get_device_name(0))

    stream = torch.cuda.Stream()
    names = [n for n in args.workloads.split(",") if n]
    results, baselines = {}, {}
    with torch.cuda.stream(stream):
        for name in names:
            results[name], baselines[name] = run_workload(torch, lcca, synth, name, args, not args.no_oracle,
                                                          args.cpu_seconds if name == names[0] else 0.0,
                                                          bf16_variant=name == names[0] and not args.no_bf16_variant)

    head = names[0]
    r = results[head]
    for n, e in r["stages"].items():
        e["traffic"] = measured_traffic(head, n)
    # the dominant kernel of the headline workload: the stage with the most time
    dname, d = max(r["stages"].items(), key=lambda kv: kv[1]["ms"])
    traffic = d["traffic"]
    roof = {"kernel": dname, "bound": "hbm", "achieved": d["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": d["hbm_frac"], "traffic": traffic, "algorithmic_bytes": d["bytes"],
            "basis": "HIP events around the stage's C-ABI call on its launch stream: for sparse_attn_fwd the "
                     "attention kernel, the split merge and the launch gap between them (the kernel trace in "
                     "profiles/ gives each kernel's own duration)"}
    cfg = synth.CONFIGS[head]
    line = {
        "metric": METRIC, "value": round(r["rows_per_s"], 1), "unit": "query-rows/s", "n_gpus": 1,
        "steps": r["steps"], "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": head, "batch": cfg.batch, "context": cfg.total_len(0), "ratio_m": cfg.m,
                   "top_k": cfg.k, "window": cfg.window, "kv": cfg.kv_dtype, "window_cache": cfg.win_dtype,
                   "heads": cfg.H, "dim": cfg.D, "out": "f32", "cold_cache_copies": r["R"]},
        "step_hbm_GB/s": round(r["step_GB/s"], 1), "step_hbm_frac": round(r["step_hbm_frac"], 4),
        "roofline": roof,
        "cpu_baseline": baselines.get(head),
        "cpu_baseline_1t": r.get("cpu_1t"),
        "stages": r["stages"],
        "hot_rows_per_s": round(r["hot_rows_per_s"], 1) if r["hot_rows_per_s"] else None,
        "parity": r.get("parity"),
        "bf16_out": r.get("bf16_out"),
        "gated_compress": r.get("gated_compress"),
        "fp8_query": r.get("fp8_query"),
        "p_bf16": r.get("p_bf16"),
        "rope": r.get("rope"),
        "also": {n: {"rows_per_s": round(v["rows_per_s"], 1), "ms_per_step": round(v["ms_per_step"], 5),
                     "rows": v["rows"], "step_hbm_GB/s": round(v["step_GB/s"], 1),
                     "step_hbm_frac": round(v["step_hbm_frac"], 4), "step_TFLOP/s": round(v["step_TFLOP/s"], 2),
                     "hot_rows_per_s": round(v["hot_rows_per_s"], 1) if v["hot_rows_per_s"] else None,
                     "stages": v["stages"], "cold_cache_copies": v["R"], "steps": v["steps"],
                     "parity": v.get("parity"), "gated_compress": v.get("gated_compress"),
                     "fp8_query": v.get("fp8_query"), "cpu_1t": v.get("cpu_1t"),
                     "rope": v.get("rope"), "p_bf16": v.get("p_bf16")}
                 for n, v in results.items() if n != head},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
