"""Seeded synthetic workloads for compressed-KV decode and chunked prefill.

This module only draws random numbers and lays out shapes: it holds none of
the method's arithmetic (no softmax, no encoding, no attention).  Every
tensor is float32 (values) or int32 (tables, positions); turning values into
stored cache codes is left to the caller.  Each tensor has its own PCG64
stream keyed by (0x1CCA, config id, tensor id, sequence), so a tensor can be
regenerated alone and sequence by sequence.

Workloads (one attention layer each):
  tiny        fp32 throughout; 1 sequence of 1,024 tokens built by compression
              (m=4 -> 256 entries); 8 query heads, shared-KV dim 128; indexer
              4 heads x 32; top-k 64; window 128; one decode query.
  csa_64k     16 sequences x 65,536 tokens, m=4 (16,384 bf16 entries of dim
              576 per sequence), shuffled block table, 64 query heads,
              indexer 64 x 128 bf16, top-k 2,048, FP8 window of 128 tokens
              with a per-token scale; N(0,1) values with 1% outlier channels
              scaled by 8.
  hca_1m      4 sequences x 1,048,576 tokens, m=128 (8,192 bf16 entries),
              dense attention over all entries plus the FP8 window.
  prefill_8k  1 sequence: 122,880 prior tokens (30,720 entries) plus a new
              8,192-token chunk compressed and appended causally; one query
              row per new token; indexer 64 x 128; top-k 2,048; bf16 window.
  lp_512k     32 sequences x 524,288 tokens, m=4, MXFP4 entries, FP8 indexer
              keys, FP8 window, top-k 2,048.
"""
from dataclasses import dataclass, field, replace
from typing import Tuple

import numpy as np

SEED_ROOT = 0x1CCA

# tensor ids of the per-tensor streams
T_KV_ENTRIES, T_IK_ENTRIES, T_WIN, T_REM_KV, T_REM_IK, T_REM_KV_LOGIT, T_REM_IK_LOGIT = 1, 2, 3, 4, 5, 6, 7
T_NEW_KV, T_NEW_IK, T_NEW_KV_LOGIT, T_NEW_IK_LOGIT = 8, 9, 10, 11
T_Q, T_Q_IDX, T_W_IDX, T_BLOCK_PERM, T_OUTLIER = 12, 13, 14, 15, 16
T_REM_KV_GATE, T_REM_IK_GATE, T_NEW_KV_GATE, T_NEW_IK_GATE = 17, 18, 19, 20
T_ROPE_X, T_ROPE_POS = 21, 22

F32, BF16, FP8, MXFP4 = "f32", "bf16", "fp8", "mxfp4"


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    prior_len: Tuple[int, ...]      # tokens already in the cache, per sequence
    n_new: Tuple[int, ...]          # tokens appended by the step, per sequence
    m: int                          # tokens per compressed entry
    D: int                          # shared-KV dim (also the value dim unless d_v is set)
    H: int                          # query heads
    HI: int                         # indexer heads (0: dense attention, no indexer/top-k)
    dI: int                         # indexer head dim
    k: int                          # top-k
    window: int = 128
    win_cap: int = 128              # window ring capacity (>= window + new tokens - 1)
    d_v: int = 0                    # value dim; 0 -> D
    tok_dtype: str = BF16
    kv_dtype: str = BF16
    ik_dtype: str = BF16
    win_dtype: str = FP8
    q_dtype: str = BF16
    out_dtype: str = F32
    outlier_frac: float = 0.0       # fraction of channels scaled by outlier_mult
    outlier_mult: float = 8.0
    rows: str = "last"              # "last": one decode row per sequence; "new": one row per new token
    prior_sampled: bool = True      # prior entries drawn directly (else the prior is empty)
    sm_scale: float = 0.0           # 0 -> 1/sqrt(D)
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def batch(self):
        return len(self.prior_len)

    @property
    def dv(self):
        return self.d_v or self.D

    @property
    def scale(self):
        return self.sm_scale or 1.0 / np.sqrt(self.D)

    @property
    def E(self):
        return 256 // self.m

    def total_len(self, b):
        return self.prior_len[b] + self.n_new[b]

    def blocks_per_seq(self, b):
        return -(-self.total_len(b) // 256)

    @property
    def max_blocks(self):
        return max(self.blocks_per_seq(b) for b in range(self.batch))

    @property
    def num_blocks(self):
        return sum(self.blocks_per_seq(b) for b in range(self.batch))

    def rows_of(self):
        """(row_seq, row_pos) int32 arrays."""
        seq, pos = [], []
        for b in range(self.batch):
            T = self.total_len(b)
            if self.rows == "last":
                seq.append(b); pos.append(T - 1)
            else:
                for p in range(self.prior_len[b], T):
                    seq.append(b); pos.append(p)
        return np.asarray(seq, np.int32), np.asarray(pos, np.int32)

    @property
    def num_rows(self):
        return len(self.rows_of()[0])

    @property
    def max_entries(self):
        return max(self.total_len(b) // self.m for b in range(self.batch))


def _full(name, cfg_id, B, T, n_new, **kw):
    return Config(name=name, cfg_id=cfg_id, prior_len=(T - n_new,) * B, n_new=(n_new,) * B, **kw)


CONFIGS = {
    "tiny": Config(name="tiny", cfg_id=1, prior_len=(0,), n_new=(1024,), m=4, D=128, H=8, HI=4, dI=32,
                   k=64, tok_dtype=F32, kv_dtype=F32, ik_dtype=F32, win_dtype=F32, q_dtype=F32,
                   out_dtype=F32, prior_sampled=False, win_cap=128),
    "csa_64k": _full("csa_64k", 2, 16, 65536, 1, m=4, D=576, H=64, HI=64, dI=128, k=2048,
                     outlier_frac=0.01),
    "hca_1m": _full("hca_1m", 3, 4, 1048576, 1, m=128, D=576, H=64, HI=0, dI=0, k=0),
    "prefill_8k": _full("prefill_8k", 4, 1, 131072, 8192, m=4, D=576, H=64, HI=64, dI=128, k=2048,
                        win_dtype=BF16, win_cap=16384, rows="new"),
    "lp_512k": _full("lp_512k", 5, 32, 524288, 1, m=4, D=576, H=64, HI=64, dI=128, k=2048,
                     kv_dtype=MXFP4, ik_dtype=FP8),
}


def shrink(cfg: Config, name: str, prior_len, n_new, **kw) -> Config:
    """A smaller variant of a workload (same dtypes and structure)."""
    return replace(cfg, name=name, prior_len=tuple(prior_len), n_new=tuple(n_new), **kw)


# --------------------------------------------------------------------------
# random streams
# --------------------------------------------------------------------------

def rng(cfg: Config, tensor_id: int, seq: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, cfg.cfg_id, tensor_id, seq])))


def normal(cfg, tensor_id, seq, shape):
    return rng(cfg, tensor_id, seq).standard_normal(shape, dtype=np.float32)


def uniform(cfg, tensor_id, seq, shape):
    return rng(cfg, tensor_id, seq).random(shape, dtype=np.float32)


def outlier_channels(cfg: Config, dim: int, stream: int):
    """The seeded set of outlier channels of a stream (shared by queries and keys)."""
    n = int(round(cfg.outlier_frac * dim))
    if n == 0:
        return np.zeros(0, np.int64)
    return np.sort(rng(cfg, T_OUTLIER, stream).permutation(dim)[:n])


def _values(cfg, tensor_id, seq, shape, dim, stream):
    """N(0,1) float32 values with the stream's outlier channels multiplied."""
    x = normal(cfg, tensor_id, seq, shape)
    ch = outlier_channels(cfg, dim, stream)
    if ch.size:
        x[..., ch] *= np.float32(cfg.outlier_mult)
    return x


def block_table(cfg: Config):
    """[batch][max_blocks] physical block ids: a seeded permutation of all
    blocks, handed out in sequence order; unused slots hold 0."""
    perm = rng(cfg, T_BLOCK_PERM).permutation(cfg.num_blocks).astype(np.int32)
    bt = np.zeros((cfg.batch, cfg.max_blocks), np.int32)
    o = 0
    for b in range(cfg.batch):
        nb = cfg.blocks_per_seq(b)
        bt[b, :nb] = perm[o:o + nb]
        o += nb
    return bt


# --------------------------------------------------------------------------
# per-sequence tensors
# --------------------------------------------------------------------------

def prior_entries(cfg: Config, b: int):
    """Compressed entries already in the cache for sequence b (drawn directly):
    (kv [n][D], ik [n][dI] or None), n = prior_len // m."""
    n = cfg.prior_len[b] // cfg.m if cfg.prior_sampled else 0
    kv = _values(cfg, T_KV_ENTRIES, b, (n, cfg.D), cfg.D, 0)
    ik = _values(cfg, T_IK_ENTRIES, b, (n, cfg.dI), cfg.dI, 1) if cfg.HI else None
    return kv, ik


def prior_window(cfg: Config, b: int):
    """Window tokens of the prior positions still in the ring:
    (first position, [count][D])."""
    P = cfg.prior_len[b]
    t0 = max(0, P - cfg.win_cap)
    return t0, _values(cfg, T_WIN, b, (P - t0, cfg.D), cfg.D, 0)


def prior_remainder(cfg: Config, b: int):
    """Tokens of the incomplete group preceding the step (positions
    floor(P/m)*m .. P-1): (first position, kv [r][D], ik [r][dI], kv logits, ik logits)."""
    P = cfg.prior_len[b]
    t0 = (P // cfg.m) * cfg.m
    r = P - t0
    kv = _values(cfg, T_REM_KV, b, (r, cfg.D), cfg.D, 0)
    ik = _values(cfg, T_REM_IK, b, (r, cfg.dI), cfg.dI, 1) if cfg.HI else None
    a = normal(cfg, T_REM_KV_LOGIT, b, (r,))
    ai = normal(cfg, T_REM_IK_LOGIT, b, (r,)) if cfg.HI else None
    return t0, kv, ik, a, ai


def new_tokens(cfg: Config, b: int):
    """The step's new tokens of sequence b: (kv [n][D], ik [n][dI], kv logits, ik logits)."""
    n = cfg.n_new[b]
    kv = _values(cfg, T_NEW_KV, b, (n, cfg.D), cfg.D, 0)
    ik = _values(cfg, T_NEW_IK, b, (n, cfg.dI), cfg.dI, 1) if cfg.HI else None
    a = normal(cfg, T_NEW_KV_LOGIT, b, (n,))
    ai = normal(cfg, T_NEW_IK_LOGIT, b, (n,)) if cfg.HI else None
    return kv, ik, a, ai


def gate_logits(cfg: Config, b: int):
    """Per-channel aggregation logits of sequence b, N(0,1) like the
    per-token ones: (remainder-ring tokens kv [r][D], ik [r][dI]; new tokens
    kv [n][D], ik [n][dI]); the ik arrays are None without an indexer."""
    r = cfg.prior_len[b] - (cfg.prior_len[b] // cfg.m) * cfg.m
    n = cfg.n_new[b]
    rk = normal(cfg, T_REM_KV_GATE, b, (r, cfg.D))
    ri = normal(cfg, T_REM_IK_GATE, b, (r, cfg.dI)) if cfg.HI else None
    nk = normal(cfg, T_NEW_KV_GATE, b, (n, cfg.D))
    ni = normal(cfg, T_NEW_IK_GATE, b, (n, cfg.dI)) if cfg.HI else None
    return rk, ri, nk, ni


def queries(cfg: Config, b: int, nrows: int):
    """Query tensors of the rows of sequence b: (q [r][H][D], q_idx [r][HI][dI], w [r][HI])."""
    q = _values(cfg, T_Q, b, (nrows, cfg.H, cfg.D), cfg.D, 0)
    if not cfg.HI:
        return q, None, None
    qi = _values(cfg, T_Q_IDX, b, (nrows, cfg.HI, cfg.dI), cfg.dI, 1)
    w = uniform(cfg, T_W_IDX, b, (nrows, cfg.HI))
    return q, qi, w


def rope_inputs(seed: int, rows: int, heads: int, dim: int, max_pos: int):
    """Vectors to rotate and their positions: x float32 N(0,1) [rows][heads][dim],
    pos int32 [rows] uniform in [0, max_pos] with position 0 in row 0 and
    max_pos in the last row."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 0x40BE, T_ROPE_X, seed])))
    x = g.standard_normal((rows, heads, dim), dtype=np.float32)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 0x40BE, T_ROPE_POS, seed])))
    pos = g.integers(0, max_pos + 1, rows).astype(np.int32)
    if rows:
        pos[0] = 0
        pos[-1] = max_pos
    return x, pos
