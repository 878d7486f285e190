"""Plain FP64 definition of paged MLA decode (dense and top-k sparse).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No blocking, no online
softmax, no split/merge: every query row is scored against every key row it may
see, the scores go through a max-shifted exp, and the output is the weighted
sum of the value rows.

Definitions followed (citations name the page, then the section):

* MLA "MQA mode": one latent cache row per token, d_qk = 576 wide, of which the
  value is the first d_v = 512 columns; all query heads of a KV head share it
  (upstream FlashMLA README embedded in the DeepLink-org/flashmla-optimization
  page, "Support matrix" footnote [2]; "FP8 KV Cache" section for the
  512 NoPE + 64 RoPE split of a row).
* Paged cache: 64-token blocks reached through ``block_table`` (FlashMLA summary
  on sourcepulse.org, "How It Works"; FlashMLA usage page on deepep.org, the
  ``flash_mla_with_kvcache`` call and the "Block Table Manager" paragraph).
* Scores are scaled dot products, softmax over the visible keys, and the
  log-sum-exp is returned per query head (upstream README, "Return Values";
  "Sparse MLA Prefill" for the scale applied inside the scores).
* ``s_q`` query tokens per request under MTP, with a causal mask (upstream
  README "Usage / MLA Decoding"; deepep.org example passes ``causal=True``).
* Sparse decode: ``indices[b][i][k] = block * 64 + offset`` straight into the
  cache, ``-1`` invalid, no block table (upstream README, "Sparse Attention
  (indices tensor)").

Readings taken where the pages are silent:

* LSE is the natural log of the summed exp of the *scaled* scores.  (The
  sparse-prefill equations use base 2 with scores pre-multiplied by log2(e);
  that is the same quantity divided by ln 2.)
* Causal alignment is bottom-right: query i of s_q sees cache positions
  ``<= L - s_q + i``.
* A row that sees no key gets O = 0 and LSE = -inf.
* A sparse index is valid iff ``0 <= idx < num_blocks * 64``; duplicates count
  with multiplicity; block_table, seqlens and causal are ignored in sparse mode.
* The output is ``d_v`` wide (the prefill listing's ``d_qk`` output width is the
  d_qk == d_v case).
"""
from __future__ import annotations

import numpy as np

from . import fp8


def _to_f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or torch tensor (bf16 included)."""
    try:  # torch is optional for the oracle; bf16 tensors need it
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _to_i64(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to(device="cpu", dtype=torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


def ref_attend_rows(Q: np.ndarray, K: np.ndarray, dv: int, softmax_scale: float):
    """Softmax attention of query rows over key rows, value = first ``dv`` columns.

    Q: [m, d] float64, K: [n, d] float64.  Returns (O [m, dv], LSE [m]).
    Two passes: scores -> row max -> exp(s - max) -> sums -> weighted values.
    n == 0 gives O = 0, LSE = -inf.
    """
    m = Q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((m, dv)), np.full(m, -np.inf)
    S = softmax_scale * (Q @ K.T)  # [m, n]
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    Z = E.sum(axis=1)
    O = (E @ K[:, :dv]) / Z[:, None]
    lse = mx[:, 0] + np.log(Z)
    return O, lse


def visible_len(L: int, s_q: int, i: int, causal: bool) -> int:
    """Number of cache positions query ``i`` of ``s_q`` may attend (bottom-right causal)."""
    if not causal:
        return L
    return max(0, min(L, L - s_q + i + 1))


def _is_fp8(kv) -> bool:
    """An "FP8 with scale" cache: bytes, 656 per row (see ``oracle.fp8``)."""
    return str(kv.dtype) in ("uint8", "torch.uint8") and kv.shape[-1] == fp8.ROW_BYTES


def _gather_f64(kv, rows_index):
    """kv[rows_index] as float64, converting (or dequantizing) only the gathered rows."""
    try:
        import torch

        if isinstance(kv, torch.Tensor):
            ix = tuple(torch.as_tensor(np.asarray(a), dtype=torch.long) for a in rows_index)
            if _is_fp8(kv):
                return fp8.dequant_rows(kv[ix].numpy())
            return kv[ix].to(dtype=torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    if _is_fp8(kv):
        return fp8.dequant_rows(np.asarray(kv[rows_index]))
    return np.asarray(kv[rows_index], dtype=np.float64)


def _row_width(kv) -> int:
    """Values per cache row: d_qk (576 for an FP8 cache)."""
    return fp8.NOPE + fp8.ROPE if _is_fp8(kv) else kv.shape[-1]


def ref_decode_paged(q, kvcache, block_table, cache_seqlens, dv: int, causal: bool,
                     softmax_scale: float, heads=None, batches=None):
    """Dense paged MLA decode, FP64.

    q            [B, s_q, h_q, d_qk]
    kvcache      [num_blocks, page, h_kv, d_qk]   (page = 64 in every config), or
                 [num_blocks, page, h_kv, 656] uint8 in the FP8-with-scale format
                 (d_qk = 576; rows dequantized by ``oracle.fp8.dequant_rows``)
    block_table  [B, max_blocks] int; entry j of row b is the physical block of
                 logical positions [j*page, (j+1)*page) of request b
    cache_seqlens[B] int; tokens in the cache of request b (the s_q new tokens
                 included)
    heads        optional iterable of head indices to compute (default: all)
    batches      optional iterable of requests to compute (default: all)

    Returns (O [B, s_q, h_q, dv] float64, LSE [B, s_q, h_q] float64, natural
    log).  Entries not computed are NaN.  Only the cache rows a request can
    see are read (and converted to float64).
    """
    qf = _to_f64(q)
    bt = _to_i64(block_table)
    sl = _to_i64(cache_seqlens)
    B, s_q, h_q, d_qk = qf.shape
    _, page, h_kv, _ = kvcache.shape
    assert _row_width(kvcache) == d_qk and h_q % h_kv == 0 and dv <= d_qk
    group = h_q // h_kv
    head_list = list(range(h_q)) if heads is None else list(heads)
    O = np.full((B, s_q, h_q, dv), np.nan)
    LSE = np.full((B, s_q, h_q), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(sl[b])
        pos = np.arange(L)
        phys = bt[b, pos // page] if L > 0 else np.zeros(0, dtype=np.int64)
        rows = _gather_f64(kvcache, (phys, pos % page))  # [L, h_kv, d_qk], logical order
        for i in range(s_q):
            n = visible_len(L, s_q, i, causal)
            for hk in range(h_kv):
                hs = [h for h in head_list if h // group == hk]
                if not hs:
                    continue
                o, lse = ref_attend_rows(qf[b, i, hs, :], rows[:n, hk, :], dv, softmax_scale)
                O[b, i, hs, :] = o
                LSE[b, i, hs] = lse
    return O, LSE


def ref_decode_sparse(q, kvcache, indices, dv: int, softmax_scale: float, heads=None,
                      batches=None):
    """Top-k sparse MLA decode, FP64.

    q        [B, s_q, h_q, d_qk]
    kvcache  [num_blocks, page, h_kv, d_qk] (or 656-byte FP8 rows, as for dense);
             row e = block e // page, offset e % page
    indices  [B, s_q, topk] int; entry = block*page + offset, invalid if < 0 or
             >= num_blocks*page (those are dropped)
    heads    optional iterable of heads to compute (default: all); sparse decode
             computes only the first ``active_h_q`` heads.
    batches  optional iterable of requests to compute (default: all)

    Returns (O [B, s_q, h_q, dv], LSE [B, s_q, h_q]); entries not computed are NaN.
    """
    qf = _to_f64(q)
    idx = _to_i64(indices)
    B, s_q, h_q, d_qk = qf.shape
    nblk, page, h_kv, _ = kvcache.shape
    assert _row_width(kvcache) == d_qk and h_q % h_kv == 0 and dv <= d_qk
    group = h_q // h_kv
    head_list = list(range(h_q)) if heads is None else list(heads)
    O = np.full((B, s_q, h_q, dv), np.nan)
    LSE = np.full((B, s_q, h_q), np.nan)
    for b in (range(B) if batches is None else batches):
        for i in range(s_q):
            sel = idx[b, i]
            sel = sel[(sel >= 0) & (sel < nblk * page)]
            rows = _gather_f64(kvcache, (sel // page, sel % page))  # [n, h_kv, d_qk]
            for hk in range(h_kv):
                hs = [h for h in head_list if h // group == hk]
                if not hs:
                    continue
                o, lse = ref_attend_rows(qf[b, i, hs, :], rows[:, hk, :], dv, softmax_scale)
                O[b, i, hs, :] = o
                LSE[b, i, hs] = lse
    return O, LSE
