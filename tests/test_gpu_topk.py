"""topk_select on logits given directly (no indexer in front), against the
oracle's selection on the same float32 values: the index lists must be
identical.  The cases cover the selection's distinct paths: rows held in
registers and rows streamed from memory, a boundary bin small enough for the
candidate buffer and one that overflows it (all-equal rows, rows that are
mostly zero as ReLU logits can be), ties at the k-th value, negative values
and -0.0, rows of n <= k, ragged row lengths and unaligned rows."""
import numpy as np
import pytest
import torch

import oracle as O
from long_context_compressed_append_amd import lcca

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run(logits, row_pos, m, k):
    """logits float32 [rows][ld] on the host; returns device and oracle indices."""
    rows, ld = logits.shape
    dev = torch.from_numpy(logits).cuda()
    rp = torch.from_numpy(row_pos.astype(np.int32)).cuda()
    rs = torch.zeros_like(rp)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    rows_ = lcca.Rows(rs, rp, int(row_pos.max()))
    wsb = lcca.topk_workspace_size(rows_, m, k)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
    lcca.topk_select(rows_, m, dev, ld, k, idx, ws)
    torch.cuda.synchronize()
    want = O.topk(row_pos, m, logits.astype(np.float64), k)
    return idx.cpu().numpy(), want


def _check(name, logits, row_pos, m, k):
    _say("topk", name, logits.shape, "k", k)
    got, want = _run(logits, row_pos, m, k)
    bad = np.flatnonzero((got != want).any(1))
    assert bad.size == 0, "%s: rows %s differ" % (name, bad[:5])


def _relu_like(g, shape, zero_frac):
    x = np.abs(g.standard_normal(shape)).astype(np.float32) * 3.0
    x[g.random(shape) < zero_frac] = 0.0
    return x


@pytest.mark.parametrize("n", [1000, 8191, 16384, 32768, 131072, 262144])
def test_random_rows(n):
    g = np.random.default_rng(n)
    rows, m, k = 6, 4, 2048
    ld = n
    x = g.standard_normal((rows, ld)).astype(np.float32)
    # ragged lengths: the last row is full, the others shorter
    lens = np.array([n, max(1, n // 2 + 3), max(1, n - 5), max(1, k - 1), max(1, k), max(1, k + 1)])
    lens = np.minimum(lens, n)
    _check("random n=%d" % n, x, lens * m - 1, m, k)


@pytest.mark.parametrize("n", [16384, 131072])
def test_ties_zeros_and_signs(n):
    g = np.random.default_rng(7 + n)
    rows, m, k = 8, 4, 2048
    x = np.empty((rows, n), np.float32)
    x[0] = 1.25                                         # all equal: boundary bin overflows
    x[1] = _relu_like(g, n, 0.99)                       # < k nonzero: the k-th value is 0
    x[2] = _relu_like(g, n, 0.5)
    x[3] = np.round(g.standard_normal(n) * 4) / 4       # many exact ties
    x[4] = -np.abs(g.standard_normal(n)).astype(np.float32)     # all negative
    x[5] = 0.0
    x[5, ::2] = -0.0                                    # -0.0 ties +0.0
    x[5, g.integers(0, n, 100)] = 1.0
    x[6] = g.standard_normal(n).astype(np.float32) * 1e-3 + 100.0   # one narrow bin
    x[7] = g.standard_normal(n).astype(np.float32)
    x[7, g.integers(0, n, 5000)] = 3.0                  # a tie that straddles the k-th place
    _check("ties n=%d" % n, x, np.full(rows, n * m - 1), m, k)


@pytest.mark.parametrize("rows,n", [(300, 32768), (300, 5000), (100, 16384)])
def test_many_rows(rows, n):
    """The same kinds of rows, each repeated down a larger batch, with ragged
    lengths: 300 rows (more than compute units: the compact shared-memory
    layout, two rows per compute unit) and 100 rows (the full layout in one
    launch; fewer rows than that take the compact layout again)."""
    g = np.random.default_rng(17 + n + rows)
    m, k = 4, 2048
    x = np.empty((rows, n), np.float32)
    for r in range(rows):
        kind = r % 6
        if kind == 0:
            x[r] = 1.25
        elif kind == 1:
            x[r] = _relu_like(g, n, 0.99)
        elif kind == 2:
            x[r] = np.round(g.standard_normal(n) * 4) / 4
        elif kind == 3:
            x[r] = 0.0
            x[r, ::2] = -0.0
            x[r, g.integers(0, n, 100)] = 1.0
        elif kind == 4:
            x[r] = g.standard_normal(n).astype(np.float32) * 1e-3 + 100.0
        else:
            x[r] = g.standard_normal(n).astype(np.float32)
            x[r, g.integers(0, n, n // 6)] = 3.0
    lens = np.where(np.arange(rows) % 7 == 0, n, g.integers(1, n + 1, rows))
    _check("%d rows n=%d" % (rows, n), x, lens * m - 1, m, k)


def test_unaligned_rows_and_small_k():
    g = np.random.default_rng(11)
    rows, m, n = 5, 4, 20001
    ld = n + 3                                          # rows not 16-byte aligned
    x = g.standard_normal((rows, ld)).astype(np.float32)
    for k in (1, 7, 64, 4096):
        _check("unaligned k=%d" % k, x, np.array([n, n - 1, 3000, 17, 4]) * m - 1, m, k)


def test_hca_ratio():
    g = np.random.default_rng(12)
    m, n, k = 128, 8192, 512
    x = g.standard_normal((3, n)).astype(np.float32)
    _check("m=128", x, np.array([n * m - 1, n * m // 3, 5 * m]), m, k)


@pytest.mark.parametrize("k", [8192, 8193, 12000])
def test_long_rows_large_k(k):
    """Rows of 64K entries (four 16K slices, then the selection among the
    slices' candidates) with k around the 8,192 slots in which the slice and
    candidate selections stage their chosen positions before translating
    them: k = 8,192 takes the staged output, larger k the direct one; random,
    tied and ReLU-like rows, ragged lengths."""
    g = np.random.default_rng(31 + k)
    rows, m, n = 4, 4, 65536
    x = np.empty((rows, n), np.float32)
    x[0] = g.standard_normal(n).astype(np.float32)
    x[1] = np.round(g.standard_normal(n) * 4) / 4
    x[2] = _relu_like(g, n, 0.8)
    x[3] = g.standard_normal(n).astype(np.float32)
    x[3, g.integers(0, n, 20000)] = 2.0
    lens = np.array([n, n - 9, k + 5000, n // 2 + 1])
    _check("long rows k=%d" % k, x, lens * m - 1, m, k)
