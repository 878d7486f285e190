"""Sparse MLA prefill, FP64, written from its mathematical definition.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What is computed (upstream FlashMLA README embedded in the DeepLink-org/
flashmla-optimization page, "Sparse MLA Prefill": the kernel's outputs and the
PyTorch computation they are defined by).  For query token i and head h, let
T_i be the multiset of valid entries of the token's top-k list and

    z_t = sm_scale * <q[i, h, :], kv[t, 0, :]>          t in T_i   (natural units)

Then, with log2(e) converting natural units to the base-2 units the page uses,

    max_logits[i, h] = log2(e) * max_t z_t
    lse[i, h]        = log2(e) * ln sum_t exp(z_t)       (= log2 sum_t 2^(log2(e) z_t))
    out[i, h, :]     = sum_t exp(z_t) * kv[t, 0, :d_v] / sum_t exp(z_t)

i.e. softmax attention of the token's heads over its selected rows, with the
logits' maximum and log-sum-exp reported in base 2.

Readings taken where the page is silent:

* An entry is invalid if it is -1 or >= s_kv (the page's rule); invalid
  entries are left out of every sum and maximum.  A query whose entries are
  all invalid gets out = 0 and max_logits = lse = -inf.
* The value is the first d_v = 512 columns of a KV row, as in decode (the
  page's output is d_qk wide: the d_v = d_qk case).
* A duplicated index counts once per occurrence.
"""
from __future__ import annotations

import math

import numpy as np

from .decode import _to_f64, _to_i64

_LOG2E = 1.0 / math.log(2.0)


def _attend(qi: np.ndarray, rows: np.ndarray, sm_scale: float, dv: int):
    """Softmax attention of the heads qi [h_q, d] over rows [n, d] (n >= 1):
    returns (out [h_q, dv], max of the logits, natural-log LSE), per head."""
    z = sm_scale * (qi @ rows.T)                     # [h_q, n] natural-unit logits
    zmax = np.max(z, axis=1)                         # [h_q]
    w = np.exp(z - zmax[:, None])                    # unnormalised weights, <= 1
    total = np.sum(w, axis=1)                        # [h_q], >= 1
    out = (w @ rows[:, :dv]) / total[:, None]
    return out, zmax, zmax + np.log(total)


def ref_sparse_prefill(q, kv, indices, sm_scale: float, dv: int = 512, rows=None):
    """q [s_q, h_q, d_qk], kv [s_kv, h_kv=1, d_qk], indices [s_q, h_kv=1, topk].

    ``rows``: optional iterable of query tokens to compute (default: all).
    Returns (out [s_q, h_q, dv], max_logits [s_q, h_q], lse [s_q, h_q]) as
    float64, max_logits and lse in base 2; tokens not computed are NaN.
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
        entries = idx[i, 0]
        valid = entries[(entries >= 0) & (entries < s_kv)]
        if valid.size == 0:
            out[i], max_logits[i], lse[i] = 0.0, -np.inf, -np.inf
            continue
        kv_rows = _to_f64(kv[valid.tolist()])[:, 0, :]   # [n, d_qk], with multiplicity
        o, zmax, lse_e = _attend(qf[i], kv_rows, sm_scale, dv)
        out[i] = o
        max_logits[i] = _LOG2E * zmax
        lse[i] = _LOG2E * lse_e
    return out, max_logits, lse
