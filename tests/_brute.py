"""Pure-Python brute force for tiny decode problems (a pin for the oracle).

Written independently of ``oracle/``: explicit loops over requests, query
tokens, heads and cache positions, addresses resolved one token at a time
through the block table, every sum taken with ``math.fsum``.
"""
import math


def _lists(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).tolist()
    except ImportError:
        pass
    return x.tolist() if hasattr(x, "tolist") else x


def _attend(qrow, rows, dv, scale):
    if not rows:
        return [0.0] * dv, -math.inf
    scores = [scale * math.fsum(a * b for a, b in zip(qrow, r)) for r in rows]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    z = math.fsum(w)
    out = [math.fsum(w[t] * rows[t][c] for t in range(len(rows))) / z for c in range(dv)]
    return out, top + math.log(z)


def brute_paged(q, kvcache, block_table, seqlens, dv, causal, scale, heads=None):
    """Returns dict {(b, i, h): (O list, lse)}."""
    q, kv, bt, sl = _lists(q), _lists(kvcache), _lists(block_table), _lists(seqlens)
    B, s_q, h_q = len(q), len(q[0]), len(q[0][0])
    page, h_kv = len(kv[0]), len(kv[0][0])
    group = h_q // h_kv
    res = {}
    for b in range(B):
        L = int(sl[b])
        for i in range(s_q):
            if causal:
                last = L - s_q + i  # last visible position
                n = max(0, min(L, last + 1))
            else:
                n = L
            for h in (range(h_q) if heads is None else heads):
                rows = []
                for t in range(n):
                    blk = int(bt[b][t // page])
                    rows.append(kv[blk][t % page][h // group])
                res[(b, i, h)] = _attend(q[b][i][h], rows, dv, scale)
    return res


def brute_sparse(q, kvcache, indices, dv, scale, heads=None):
    q, kv, ix = _lists(q), _lists(kvcache), _lists(indices)
    B, s_q, h_q = len(q), len(q[0]), len(q[0][0])
    nblk, page, h_kv = len(kv), len(kv[0]), len(kv[0][0])
    group = h_q // h_kv
    res = {}
    for b in range(B):
        for i in range(s_q):
            for h in (range(h_q) if heads is None else heads):
                rows = []
                for e in ix[b][i]:
                    e = int(e)
                    if 0 <= e < nblk * page:
                        rows.append(kv[e // page][e % page][h // group])
                res[(b, i, h)] = _attend(q[b][i][h], rows, dv, scale)
    return res
