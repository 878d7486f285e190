"""Pins of the sparse-prefill oracle (``oracle.prefill.ref_sparse_prefill``).

* A pure-Python brute force of the page's equations (loops and math.fsum) on
  tiny inputs with invalid entries of both kinds (-1 and >= s_kv) and
  duplicates.
* Closed forms: q = 0 gives the mean of the selected value rows, lse =
  log2(n) and max_logits = 0; a single valid index gives that row's value,
  lse = max_logits = its logit.
* All-invalid queries give out = 0 and lse = max_logits = -inf.
* The same quantities as the sparse decode oracle (pinned on its own): equal
  out, lse_decode = lse_prefill * ln 2.
"""
import math

import numpy as np
import torch

import oracle
from oracle.prefill import ref_sparse_prefill


def _case(seed, s_q=3, h_q=4, s_kv=50, d=12, topk=9):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((s_q, h_q, d))
    kv = rng.standard_normal((s_kv, 1, d))
    idx = rng.integers(-3, s_kv + 4, size=(s_q, 1, topk)).astype(np.int32)
    idx[0, 0, :2] = idx[0, 0, 2]  # duplicates
    return q, kv, idx


def _brute(q, kv, idx, scale, dv):
    s_q, h_q, d = q.shape
    s_kv = kv.shape[0]
    out = np.zeros((s_q, h_q, dv))
    mx = np.zeros((s_q, h_q))
    lse = np.zeros((s_q, h_q))
    for i in range(s_q):
        sel = [int(t) for t in idx[i, 0] if 0 <= t < s_kv]
        for h in range(h_q):
            if not sel:
                mx[i, h] = lse[i, h] = -math.inf
                continue
            P = [math.fsum(q[i, h, c] * kv[t, 0, c] for c in range(d)) * scale * math.log2(math.e)
                 for t in sel]
            m = max(P)
            l2 = m + math.log2(math.fsum(2.0 ** (p - m) for p in P))
            mx[i, h], lse[i, h] = m, l2
            for c in range(dv):
                out[i, h, c] = math.fsum(2.0 ** (p - l2) * kv[t, 0, c] for p, t in zip(P, sel))
    return out, mx, lse


def test_matches_brute_force():
    for seed in (1, 2, 3):
        q, kv, idx = _case(seed)
        o, m, l = ref_sparse_prefill(q, kv, idx, 0.3, dv=8)
        bo, bm, bl = _brute(q, kv, idx, 0.3, 8)
        assert np.allclose(o, bo, rtol=0, atol=1e-12)
        assert np.allclose(m, bm, rtol=0, atol=1e-12)
        assert np.allclose(l, bl, rtol=0, atol=1e-12)


def test_zero_query_closed_form():
    q, kv, idx = _case(4)
    q[:] = 0
    o, m, l = ref_sparse_prefill(q, kv, idx, 0.5, dv=12)
    for i in range(q.shape[0]):
        sel = [t for t in idx[i, 0] if 0 <= t < kv.shape[0]]
        assert np.allclose(o[i], kv[sel, 0, :].mean(axis=0), atol=1e-13)
        assert np.allclose(l[i], math.log2(len(sel)), atol=1e-13)
        assert np.all(m[i] == 0)


def test_single_valid_index_and_all_invalid():
    q, kv, idx = _case(5)
    idx[:] = -1
    idx[1, 0, 3] = 7
    idx[2, 0, :] = kv.shape[0] + 2  # past s_kv: invalid
    o, m, l = ref_sparse_prefill(q, kv, idx, 0.25, dv=12)
    logit = q[1] @ kv[7, 0] * 0.25 * math.log2(math.e)
    assert np.allclose(o[1], np.broadcast_to(kv[7, 0], (q.shape[1], 12)), atol=1e-14)
    assert np.allclose(m[1], logit, atol=1e-13) and np.allclose(l[1], logit, atol=1e-13)
    for i in (0, 2):
        assert np.all(o[i] == 0) and np.all(np.isneginf(m[i])) and np.all(np.isneginf(l[i]))


def test_same_quantities_as_sparse_decode_oracle():
    q, kv, idx = _case(6, s_q=4, h_q=3, s_kv=128, d=16, topk=20)
    # decode view: batch = s_q, one query token each, 64-row pages
    kv4 = torch.from_numpy(kv.reshape(2, 64, 1, 16))
    idx_dec = idx.copy()
    idx_dec[idx_dec >= kv.shape[0]] = -1
    o_d, l_d = oracle.ref_decode_sparse(torch.from_numpy(q[:, None]), kv4,
                                        torch.from_numpy(idx_dec), 10, 0.2)
    o, m, l = ref_sparse_prefill(q, kv, idx, 0.2, dv=10)
    assert np.allclose(o, o_d[:, 0], atol=1e-13)
    assert np.allclose(l * math.log(2), l_d[:, 0], atol=1e-13)
