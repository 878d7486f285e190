"""Sparse MLA prefill, FP64, in the order of the pages' equivalent code.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Definition (upstream FlashMLA README embedded in the DeepLink-org/
flashmla-optimization page, "Sparse MLA Prefill", the PyTorch code the kernel
is equivalent to): for query token i with its top-k KV rows K_i = kv[indices[i]],

    P          = (Q_i @ K_i^T) * sm_scale * log2(e)      [h_q, topk]
    max_logits = max over the top-k of P                  [h_q]
    lse        = log2 sum 2^P                             [h_q]  (base 2)
    S          = 2^(P - lse)
    out        = S @ K_i                                  [h_q, d_v]

Readings taken where the page is silent:

* Invalid entries (-1 or >= s_kv, the page's rule) are left out of every sum
  and maximum; a query whose entries are all invalid gets out = 0 and
  max_logits = lse = -inf.
* The value is the first d_v = 512 columns of a KV row, as in decode (the
  printed ``S @ focused_kv`` is d_qk wide, the d_v = d_qk case).
* Duplicated indices count once per occurrence.
"""
from __future__ import annotations

import math

import numpy as np

from .decode import _to_f64, _to_i64


def ref_sparse_prefill(q, kv, indices, sm_scale: float, dv: int = 512, rows=None):
    """q [s_q, h_q, d_qk], kv [s_kv, h_kv=1, d_qk], indices [s_q, h_kv=1, topk].

    ``rows``: optional iterable of query tokens to compute (default: all).
    Returns (out [s_q, h_q, dv], max_logits [s_q, h_q], lse [s_q, h_q]) as
    float64, lse in base 2; tokens not computed are NaN.
    """
    qf = _to_f64(q)
    idx = _to_i64(indices)
    s_q, h_q, d_qk = qf.shape
    s_kv, h_kv, d_kv = kv.shape
    assert h_kv == 1 and d_kv == d_qk and dv <= d_qk and idx.shape[:2] == (s_q, 1)
    out = np.full((s_q, h_q, dv), np.nan)
    max_logits = np.full((s_q, h_q), np.nan)
    lse = np.full((s_q, h_q), np.nan)
    for i in (range(s_q) if rows is None else rows):
        sel = idx[i, 0]
        sel = sel[(sel >= 0) & (sel < s_kv)]
        if sel.size == 0:
            out[i] = 0.0
            max_logits[i] = -np.inf
            lse[i] = -np.inf
            continue
        focused = _to_f64(kv[sel.tolist()])[:, 0, :]               # [n, d_qk]
        P = (qf[i] @ focused.T) * sm_scale * math.log2(math.e)    # [h_q, n]
        mx = P.max(axis=1)
        l2 = mx + np.log2(np.exp2(P - mx[:, None]).sum(axis=1))  # log2 sum 2^P
        S = np.exp2(P - l2[:, None])
        out[i] = S @ focused[:, :dv]
        max_logits[i] = mx
        lse[i] = l2
    return out, max_logits, lse
