"""40-digit decimal brute force for tiny inputs (stdlib only).

An implementation of the four stages written directly from their plain
definitions, independent of the C oracle, used to pin it:
  * group compression: softmax over the group's per-token logits, then the
    weighted sum of the token vectors;
  * indexer logit: sum over heads of weight * ReLU(q_h . k), times s_I;
  * top-k: the subset of size k with the largest logit sum, ties resolved
    towards smaller entry indices (exhaustive over subsets);
  * attention: softmax of scaled dot products over the key list, weighted
    sum of the values, log-sum-exp.
"""
from decimal import Decimal, getcontext
from itertools import combinations

getcontext().prec = 40


def D(x):
    return Decimal(float(x))


def softmax_weights(a):
    a = [D(v) for v in a]
    e = [v.exp() for v in a]
    s = sum(e, Decimal(0))
    return [v / s for v in e]


def compress(x, a):
    """x: [m][dim] floats, a: [m] floats -> [dim] Decimals."""
    w = softmax_weights(a)
    dim = len(x[0])
    return [sum((w[i] * D(x[i][d]) for i in range(len(x))), Decimal(0)) for d in range(dim)]


def index_logit(q, w, key, s_I=1.0):
    """q: [HI][dI], w: [HI], key: [dI] -> Decimal."""
    tot = Decimal(0)
    for h in range(len(q)):
        dot = sum((D(q[h][d]) * D(key[d]) for d in range(len(key))), Decimal(0))
        tot += D(w[h]) * max(dot, Decimal(0))
    return D(s_I) * tot


def topk_subset(logits, k):
    """Exhaustive: the size-min(k, n) subset maximising the logit sum; among
    maximisers the one whose sorted index list is lexicographically smallest.
    This equals ranking by (value desc, index asc) when values are distinct
    and breaks equal values towards smaller indices."""
    n = len(logits)
    k = min(k, n)
    vals = [D(v) for v in logits]
    best, best_sum = None, None
    for sub in combinations(range(n), k):      # lexicographic order
        s = sum((vals[i] for i in sub), Decimal(0))
        if best is None or s > best_sum:
            best, best_sum = sub, s
    return list(best)


def attention(q, keys, d_v, scale):
    """q: [H][Dm], keys: [n][Dm] (value = key[:d_v]) -> (o [H][d_v], lse [H])."""
    outs, lses = [], []
    sc = D(scale)
    for qh in q:
        s = [sc * sum((D(qh[d]) * D(k[d]) for d in range(len(k))), Decimal(0)) for k in keys]
        M = max(s)
        e = [(v - M).exp() for v in s]
        den = sum(e, Decimal(0))
        outs.append([sum((e[j] * D(keys[j][d]) for j in range(len(keys))), Decimal(0)) / den
                     for d in range(d_v)])
        lses.append(M + den.ln())
    return outs, lses
