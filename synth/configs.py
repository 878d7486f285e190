"""Seeded input recipes for paged MLA decode (no attention arithmetic here).

Recipe (shared by every config):

* RNG ``numpy.random.Generator(PCG64(seed))``; the five named workloads use
  seed ``1000 + k`` for workload k.
* Draw order: sequence lengths -> block permutation -> q -> kvcache ->
  sparse index positions.
* Values are float32 standard normals rounded once to bfloat16 (round to
  nearest even, by torch's cast), drawn in chunks of 2**24 values; fp16
  cases round the same draws to fp16 instead.
* Logical block j of request b lives in physical block ``block_table[b][j]``.
  Physical blocks are a random permutation of the pool, handed out in batch
  order; table entries past a request's last block are -1 (except the tiny
  workload, whose table is the whole permutation reshaped).
* Sparse indices are ``block * 64 + offset`` of sorted distinct positions,
  with a tail of the sorted list replaced by -1.
* FP8 caches ("FP8 with scale", 656-byte rows: 512 e4m3, 4 fp32 scales, 64
  bf16): the row's 576 values are float32 standard normals (times 2^u per row,
  u ~ U[-spread, spread], when asked); each group of 128 NoPE values gets the
  scale amax / 448 (1 for an all-zero group) and is cast to float8_e4m3fn by
  torch (nearest even); the 64 RoPE values are rounded to bfloat16.  This is
  input preparation only -- the decode reads whatever bytes the cache holds.
"""
from __future__ import annotations

import math

import numpy as np
import torch

PAGE = 64
CHUNK = 1 << 24


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_from_f32(a: np.ndarray) -> torch.Tensor:
    """Round float32 values to bfloat16 (RNE) as a CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def normal_bf16(rng: np.random.Generator, shape, dtype=torch.bfloat16) -> torch.Tensor:
    """Float32 standard normals rounded once to ``dtype`` (bf16, or fp16)."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=dtype)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        out[s:e] = torch.from_numpy(rng.standard_normal(e - s, dtype=np.float32)).to(dtype)
    return out.view(*shape)


FP8_ROW = 656


def fp8_rows(rng: np.random.Generator, n_rows: int, spread: float = 0.0) -> torch.Tensor:
    """``n_rows`` FP8-with-scale cache rows as a uint8 tensor [n_rows, 656]."""
    out = torch.empty((n_rows, FP8_ROW), dtype=torch.uint8)
    per = max(1, CHUNK // 576)
    for s in range(0, n_rows, per):
        e = min(n_rows, s + per)
        x = rng.standard_normal((e - s, 576), dtype=np.float32)
        if spread:
            x *= np.exp2(rng.uniform(-spread, spread, size=(e - s, 1))).astype(np.float32)
        g = x[:, :512].reshape(e - s, 4, 128)
        amax = np.abs(g).max(axis=2)
        scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        codes = torch.from_numpy(np.ascontiguousarray(g / scale[:, :, None]).reshape(e - s, 512))
        out[s:e, :512] = codes.to(torch.float8_e4m3fn).view(torch.uint8)
        out[s:e, 512:528] = torch.from_numpy(scale.view(np.uint8).reshape(e - s, 16))
        rope = bf16_from_f32(x[:, 512:]).view(torch.uint8).reshape(e - s, 128)
        out[s:e, 528:] = rope
    return out


def _table_from_perm(perm: np.ndarray, nblocks: np.ndarray, width: int) -> np.ndarray:
    table = np.full((len(nblocks), width), -1, dtype=np.int32)
    cur = 0
    for b, n in enumerate(nblocks):
        table[b, :n] = perm[cur:cur + n]
        cur += n
    return table


def make_dense_case(seed: int, *, B: int, s_q: int, h_q: int, seqlens=None,
                    seqlen_sampler=None, d_qk: int = 576, d_v: int = 512, h_kv: int = 1,
                    causal: bool = False, spare_frac: float = 0.0, table_width=None,
                    reshape_table: bool = False, name: str = "dense", kv_fp8: bool = False,
                    fp8_spread: float = 0.0, dtype=torch.bfloat16) -> dict:
    """A dense paged-decode case.  ``seqlens`` fixed, or drawn by ``seqlen_sampler(rng)``.
    ``kv_fp8``: the cache is FP8 with scale (d_qk must be 576)."""
    assert not kv_fp8 or d_qk == 576
    rng = rng_for(seed)
    if seqlens is None:
        seqlens = np.asarray(seqlen_sampler(rng), dtype=np.int64)
    seqlens = np.asarray(seqlens, dtype=np.int64)
    assert len(seqlens) == B
    nblocks = (seqlens + PAGE - 1) // PAGE
    n_used = int(nblocks.sum())
    spare = int(math.ceil(spare_frac * n_used))
    if reshape_table:
        width = int(table_width)
        pool = B * width
        perm = rng.permutation(pool).astype(np.int32)
        table = perm.reshape(B, width).copy()
    else:
        pool = max(1, n_used + spare)
        width = int(table_width) if table_width is not None else max(1, int(nblocks.max(initial=0)))
        perm = rng.permutation(pool).astype(np.int32)
        table = _table_from_perm(perm, nblocks, width)
    q = normal_bf16(rng, (B, s_q, h_q, d_qk), dtype)
    if kv_fp8:
        kv = fp8_rows(rng, pool * PAGE * h_kv, fp8_spread).view(pool, PAGE, h_kv, FP8_ROW)
    else:
        kv = normal_bf16(rng, (pool, PAGE, h_kv, d_qk), dtype)
    return dict(
        name=name, sparse=False, q=q, kvcache=kv, kv_fp8=kv_fp8,
        block_table=torch.from_numpy(table),
        cache_seqlens=torch.from_numpy(seqlens.astype(np.int32)),
        indices=None, s_q=s_q, h_q=h_q, h_kv=h_kv, d_qk=d_qk, d_v=d_v,
        causal=bool(causal), softmax_scale=float(d_qk) ** -0.5,
        active_h_q=h_q, topk=0,
    )


def make_sparse_case(seed: int, *, B: int, s_q: int, h_q: int, active_h_q: int,
                     topk: int, cache_len: int, invalid_tail: int, d_qk: int = 512,
                     d_v: int = 512, h_kv: int = 1, name: str = "sparse", kv_fp8: bool = False,
                     fp8_spread: float = 0.0, dtype=torch.bfloat16) -> dict:
    """A top-k sparse-decode case: every request owns ``cache_len`` tokens of a
    shared pool; each query token draws ``topk`` distinct positions, sorted,
    and the last ``invalid_tail`` entries become -1."""
    rng = rng_for(seed)
    width = (cache_len + PAGE - 1) // PAGE
    pool = B * width
    perm = rng.permutation(pool).astype(np.int32)
    table = perm.reshape(B, width)
    assert not kv_fp8 or d_qk == 576
    q = normal_bf16(rng, (B, s_q, h_q, d_qk), dtype)
    if kv_fp8:
        kv = fp8_rows(rng, pool * PAGE * h_kv, fp8_spread).view(pool, PAGE, h_kv, FP8_ROW)
    else:
        kv = normal_bf16(rng, (pool, PAGE, h_kv, d_qk), dtype)
    idx = np.empty((B, s_q, topk), dtype=np.int32)
    for b in range(B):
        for i in range(s_q):
            pos = np.sort(rng.choice(cache_len, size=topk, replace=False))
            row = table[b, pos // PAGE].astype(np.int64) * PAGE + pos % PAGE
            if invalid_tail:
                row[topk - invalid_tail:] = -1
            idx[b, i] = row
    return dict(
        name=name, sparse=True, q=q, kvcache=kv, kv_fp8=kv_fp8,
        block_table=torch.from_numpy(table.copy()),
        cache_seqlens=torch.full((B,), cache_len, dtype=torch.int32),
        indices=torch.from_numpy(idx), s_q=s_q, h_q=h_q, h_kv=h_kv, d_qk=d_qk,
        d_v=d_v, causal=False, softmax_scale=float(d_qk) ** -0.5,
        active_h_q=active_h_q, topk=topk,
    )


def make_prefill_case(seed: int, *, s_q: int, s_kv: int, h_q: int, topk: int, d_qk: int = 576,
                      d_v: int = 512, invalid_tail: int = 0, past_end: int = 0,
                      name: str = "sparse prefill", dtype=torch.bfloat16) -> dict:
    """A sparse-prefill case: q [s_q, h_q, d_qk], kv [s_kv, 1, d_qk] bf16
    normals; query i draws ``topk`` distinct positions of [0, s_kv), sorted;
    the last ``invalid_tail`` become -1 and the ``past_end`` before them
    become s_kv + j (also invalid)."""
    rng = rng_for(seed)
    q = normal_bf16(rng, (s_q, h_q, d_qk), dtype)
    kv = normal_bf16(rng, (s_kv, 1, d_qk), dtype)
    idx = np.empty((s_q, 1, topk), dtype=np.int32)
    for i in range(s_q):
        row = np.sort(rng.choice(s_kv, size=topk, replace=False)).astype(np.int64)
        if invalid_tail:
            row[topk - invalid_tail:] = -1
        if past_end:
            lo = topk - invalid_tail - past_end
            row[lo:topk - invalid_tail] = s_kv + np.arange(past_end)
        idx[i, 0] = row
    return dict(name=name, prefill=True, q=q, kv=kv, indices=torch.from_numpy(idx), s_q=s_q,
                s_kv=s_kv, h_q=h_q, topk=topk, d_qk=d_qk, d_v=d_v,
                softmax_scale=float(d_qk) ** -0.5)


# Sparse prefill: one 4096-token chunk over a 32768-token context, every query
# with its own top-2048 positions (DeepSeek-style sparse attention shapes: 128
# heads, 576-wide latent rows).
PREFILL_WORKLOAD = dict(name="sparse prefill: s_q=4096 s_kv=32768 h_q=128 d_qk=576 d_v=512 topk 2048",
                      s_q=4096, s_kv=32768, h_q=128, topk=2048)


def _c2_lens(rng):
    return rng.integers(1, 4097, size=64)


def _skewed_long_lens(rng):
    lo, hi = math.log(32768), math.log(131072)
    long = np.floor(np.exp(rng.uniform(lo, hi, size=8))).astype(np.int64)
    long = np.clip(long, 32768, 131072)
    short = rng.integers(1, 257, size=8)
    return np.concatenate([long, short])


WORKLOADS = {
    1: dict(name="tiny: B=2 s_q=1 h_q=16 seqlens {64,200} pool 8",
            kind="dense", B=2, s_q=1, h_q=16, seqlens=[64, 200], table_width=4,
            reshape_table=True),
    2: dict(name="varlen: B=64 s_q=1 h_q=128 seqlens U[1,4096] +10% spare blocks",
            kind="dense", B=64, s_q=1, h_q=128, seqlen_sampler=_c2_lens, spare_frac=0.1,
            table_width=64),
    3: dict(name="MTP: B=128 s_q=2 causal h_q=128 seqlens 4096",
            kind="dense", B=128, s_q=2, h_q=128, seqlens=[4096] * 128, causal=True,
            table_width=64),
    4: dict(name="skewed long context: B=16 s_q=1 h_q=64, 8 x logU[32k,128k] + 8 x U[1,256]",
            kind="dense", B=16, s_q=1, h_q=64, seqlen_sampler=_skewed_long_lens, table_width=2048),
    5: dict(name="top-k sparse: B=32 s_q=1 h_q=64 (16 active) d_qk=d_v=512 topk 2048, 102 invalid",
            kind="sparse", B=32, s_q=1, h_q=64, active_h_q=16, topk=2048, cache_len=65536,
            invalid_tail=102, d_qk=512, d_v=512),
}


# The same shapes with an FP8-with-scale cache (576-wide rows: the format holds
# 512 + 64 values), seed 1000 + k as for the bf16 workload they follow.
FP8_WORKLOADS = {
    "4f": dict(WORKLOADS[4], name="skewed long context, FP8 cache: B=16 s_q=1 h_q=64, "
                                "8 x logU[32k,128k] + 8 x U[1,256]", kv_fp8=True),
    "5f": dict(WORKLOADS[5], name="top-k sparse, FP8 cache: B=32 s_q=1 h_q=64 (16 active) "
                                "d_qk=576 d_v=512 topk 2048, 102 invalid", d_qk=576, kv_fp8=True),
}


def make_config(k) -> dict:
    """The five named workloads (k = 1..5), seed 1000 + k, their FP8-cache
    variants ("4f", "5f") and the sparse prefill chunk ("p", seed 1100)."""
    if k == "p":
        return make_prefill_case(1100, **PREFILL_WORKLOAD)
    if isinstance(k, str) and k in FP8_WORKLOADS:
        spec = dict(FP8_WORKLOADS[k])
        seed = 1000 + int(k[:-1])
    else:
        k = int(k)
        spec = dict(WORKLOADS[k])
        seed = 1000 + k
    kind = spec.pop("kind")
    name = spec.pop("name")
    if kind == "dense":
        return make_dense_case(seed, name=name, **spec)
    return make_sparse_case(seed, name=name, **spec)


def make_case(kind: str, seed: int, **kw) -> dict:
    return make_dense_case(seed, **kw) if kind == "dense" else make_sparse_case(seed, **kw)
