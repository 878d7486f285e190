"""GPU parity of the FP8-with-scale KV cache path against the FP64 oracle.

The cache rows are 656 bytes (512 e4m3 + 4 fp32 scales + 64 bf16 RoPE); the
oracle dequantizes them by their definition (``oracle.fp8``) and runs the same
FP64 attention as for bf16 caches.  Tolerances are those of the bf16 parity
tests.  Cases: ragged multi-tile dense decode (causal and not, several head
counts and forced split counts), widely varying scales, sparse decode with
invalid indices and active heads, NaN-poisoned bytes outside what a request
may see, the split-KV + combine stages, the skewed long-context workload at
full size (sampled requests) and the top-k sparse shape with a 576-wide FP8
cache, sparse pools past 4 GiB (64-bit row addressing) and between 2 and 4
GiB (32-bit unsigned row offsets above 2^31).
"""
import numpy as np
import pytest
import torch

import mla_paged_kv_amd as mla
from synth.configs import WORKLOADS, _skewed_long_lens, make_dense_case, make_sparse_case
from tests._gpu_util import compare, log, metadata, run_gpu, run_oracle, to_device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"libmla: {mla.lib_path()}  device: {torch.cuda.get_device_name(0)}")


def _check(case, num_parts=0, heads=None, batches=None, what=""):
    log(f"case {what}: num_parts={num_parts}")
    d = to_device(case)
    meta = metadata(case, num_parts=num_parts)
    out, lse = run_gpu(d, meta)
    O, LSE = to_np(out, lse)
    O_ref, LSE_ref = run_oracle(case, heads=heads, batches=batches)
    compare(O, LSE, O_ref, LSE_ref, what)
    return meta, out, lse


@pytest.mark.parametrize("s_q,causal,h_q", [(1, False, 16), (2, True, 64), (1, False, 128),
                                            (3, True, 8)])
def test_fp8_dense_ragged_multi_tile(s_q, causal, h_q):
    lens = [1, 63, 64, 65, 700, 2, 130]
    case = make_dense_case(801, B=len(lens), s_q=s_q, h_q=h_q, seqlens=lens, causal=causal,
                           spare_frac=0.2, kv_fp8=True)
    for P in (0, 1, 5, 37):
        _check(case, num_parts=P, what=f"fp8 ragged s_q={s_q} causal={causal} h_q={h_q} P={P}")


def test_fp8_scales_spanning_many_binades():
    case = make_dense_case(803, B=3, s_q=1, h_q=32, seqlens=[900, 64, 1500], kv_fp8=True,
                           fp8_spread=8.0)
    for P in (0, 7):
        _check(case, num_parts=P, what=f"fp8 spread P={P}")


@pytest.mark.parametrize("active,P", [(16, 0), (64, 5), (32, 1)])
def test_fp8_sparse(active, P):
    case = make_sparse_case(805, B=4, s_q=2, h_q=64, active_h_q=active, topk=1024,
                            cache_len=6000, invalid_tail=37, d_qk=576, kv_fp8=True)
    _check(case, num_parts=P, what=f"fp8 sparse active={active} P={P}")


@pytest.mark.parametrize("h_q", [16, 8])
def test_fp8_poisoned_bytes_do_not_leak(h_q):
    """NaN codes and NaN scales in rows a request may not see (page tails,
    spare pages) leave the result bit-identical (h_q = 16: units of 32 rows,
    the pair kernel; h_q = 8: 16 rows, the narrow kernel)."""
    case = make_dense_case(807, B=3, s_q=2, h_q=h_q, seqlens=[70, 129, 1], causal=True,
                           spare_frac=1.0, kv_fp8=True)
    d = to_device(case)
    meta = metadata(case, num_parts=4)
    o1, l1 = run_gpu(d, meta)
    kv = case["kvcache"].clone()
    used = set()
    for b, L in enumerate(case["cache_seqlens"].tolist()):
        nb = (L + 63) // 64
        for j in range(nb):
            blk = int(case["block_table"][b, j])
            used.add(blk)
            if j == nb - 1 and L % 64:
                kv[blk, L % 64:] = 0x7F  # NaN codes, NaN scales, NaN RoPE
    for blk in range(kv.shape[0]):
        if blk not in used:
            kv[blk] = 0xFF
    bt = case["block_table"].clone()
    bt[bt < 0] = 0
    o2, l2 = run_gpu(dict(d, kvcache=kv.cuda(), block_table=bt.cuda()), meta)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O, LSE = to_np(o2, l2)
    compare(O, LSE, *run_oracle(case), "fp8 poisoned")


def test_fp8_sparse_poisoned_rows_do_not_leak():
    case = make_sparse_case(809, B=2, s_q=1, h_q=16, active_h_q=16, topk=256, cache_len=2048,
                            invalid_tail=40, d_qk=576, kv_fp8=True)
    d = to_device(case)
    meta = metadata(case, num_parts=3)
    o1, l1 = run_gpu(d, meta)
    kv = case["kvcache"].clone().view(-1, 656)
    keep = torch.zeros(kv.shape[0], dtype=torch.bool)
    iv = case["indices"].flatten()
    keep[iv[iv >= 0].long()] = True
    kv[~keep] = 0x7F
    o2, l2 = run_gpu(dict(d, kvcache=kv.view_as(case["kvcache"]).cuda()), meta)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_stages_compose_to_decode():
    case = make_dense_case(811, B=3, s_q=1, h_q=64, seqlens=[3000, 70, 900], kv_fp8=True)
    d = to_device(case)
    meta = metadata(case, num_parts=9)
    assert meta.num_split_units > 0
    o1, l1 = run_gpu(d, meta)
    out, lse, ws = mla.mla_decode_paged(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"],
                                        512, meta, softmax_scale=case["softmax_scale"], stage="split")
    mla.mla_combine(meta, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, out) and torch.equal(l1, lse)


def test_fp8_pages_call_shape():
    """flash_mla_with_kvcache(..., is_fp8_kvcache=True) on a float8 view of the cache."""
    case = make_dense_case(813, B=2, s_q=1, h_q=16, seqlens=[500, 33], kv_fp8=True)
    d = to_device(case)
    meta, ns = mla.get_mla_metadata(d["cache_seqlens"], 16, 1, is_fp8_kvcache=True)
    out, lse = mla.flash_mla_with_kvcache(d["q"], d["kvcache"].view(torch.float8_e4m3fn),
                                          d["block_table"], d["cache_seqlens"], 512, meta, ns,
                                          is_fp8_kvcache=True)
    torch.cuda.synchronize()
    O, LSE = to_np(out, lse)
    compare(O, LSE, *run_oracle(case), "fp8 pages call")


def test_fp8_skewed_long_context_full_size():
    spec = dict(WORKLOADS[4])
    case = make_dense_case(1004, B=16, s_q=1, h_q=64, seqlen_sampler=_skewed_long_lens, table_width=2048,
                           kv_fp8=True)
    log(f"fp8 skewed long context: {spec['name']}")
    _check(case, num_parts=0, batches=[0, 3, 7, 8, 12, 15], what="fp8 skewed long context")


def test_fp8_sparse_topk2048_full_size():
    case = make_sparse_case(1005, B=32, s_q=1, h_q=64, active_h_q=16, topk=2048, cache_len=65536,
                            invalid_tail=102, d_qk=576, kv_fp8=True)
    _check(case, num_parts=0, batches=list(range(0, 32, 5)), what="fp8 sparse topk 2048")


def _sparse_big_pool(fp8, h_q, gib):
    """A sparse call over a pool of about `gib` GiB whose selected rows include
    the pool's last 200000 (and a few invalid indices)."""
    row_bytes = 656 if fp8 else 1152
    d_qk = 576
    n_rows = (int(gib * 2 ** 30) // row_bytes // 64 + 1) * 64
    rng = np.random.default_rng(815)
    B, topk = 2, 300
    pos = np.sort(rng.choice(n_rows, size=(B, topk), replace=True), axis=1).astype(np.int64)
    pos[:, -50:] = np.sort(rng.integers(n_rows - 200000, n_rows, size=(B, 50)), axis=1)
    pos[0, :5] = -1
    used = np.unique(pos[pos >= 0])
    # small case with the same selected rows, then placed into the big pool
    src = make_sparse_case(817, B=1, s_q=1, h_q=h_q, active_h_q=h_q, topk=64,
                           cache_len=len(used) + 64, invalid_tail=0, d_qk=d_qk, kv_fp8=fp8)
    rows_small = src["kvcache"].reshape(-1, src["kvcache"].shape[-1])[:len(used)]
    log(f"pool of {n_rows} rows ({n_rows * row_bytes / 2**30:.2f} GiB), fp8={fp8}")
    shape = (n_rows // 64, 64, 1, row_bytes if fp8 else d_qk)
    kv_cpu = torch.zeros(shape, dtype=torch.uint8 if fp8 else torch.bfloat16)
    flat = kv_cpu.view(-1, shape[-1])
    flat[torch.from_numpy(used)] = rows_small
    q = src["q"][:1].expand(B, 1, h_q, d_qk).contiguous()
    idx = torch.from_numpy(pos.reshape(B, 1, topk).astype(np.int32))
    case = dict(src, q=q, kvcache=kv_cpu, indices=idx, topk=topk, active_h_q=h_q,
                cache_seqlens=torch.full((B,), n_rows, dtype=torch.int32))
    d = dict(case, q=q.cuda(), kvcache=kv_cpu.cuda(), indices=idx.cuda())
    meta = metadata(case, num_parts=0)
    out, lse = run_gpu(d, meta)
    O, LSE = to_np(out, lse)
    compare(O, LSE, *run_oracle(case), f"pool of {gib} GiB fp8={fp8} h_q={h_q}")
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fp8,h_q", [(False, 16), (True, 16), (False, 128)])
def test_sparse_pool_past_4gib(fp8, h_q):
    """Rows beyond byte offset 2^32 of the pool: the 64-bit addressing path."""
    _sparse_big_pool(fp8, h_q, 4.6)


@pytest.mark.parametrize("fp8,h_q", [(False, 16), (True, 16), (False, 128)])
def test_sparse_pool_between_2_and_4_gib(fp8, h_q):
    """Rows beyond byte offset 2^31 of a pool below 4 GiB: the 32-bit buffer
    offsets, which must be unsigned there."""
    _sparse_big_pool(fp8, h_q, 3.3)
