"""GPU parity: the HIP path (through the C-ABI binding) against the FP64 oracle.

Small cases are compared on every output; the five named workloads run at full
size in the launch configuration the benchmark uses (default part count),
compared on every request.  Units of more than 64 query rows run on the decode
kernel (128 rows per workgroup), smaller ones on the pair kernel; both are
covered, dense and sparse.  Edge cases: empty and one-token caches,
exact page multiples, causal rows that see nothing, NaN-poisoned tails and
spare blocks, invalid and duplicate sparse indices, forced split counts from 1
to past 64 per request, run-to-run and block-permutation bit identity, and
active-head-only runs against all-head runs.
"""
import numpy as np
import pytest
import torch

from synth.configs import make_config, make_dense_case, make_sparse_case
from tests._gpu_util import compare, log, metadata, run_gpu, run_oracle, to_device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_amd as mla
    log(f"libmla: {mla.lib_path()}  device: {torch.cuda.get_device_name(0)}")


def _check(case, num_parts=0, heads=None, batches=None, what=""):
    log(f"case {what or case.get('name')}: num_parts={num_parts}")
    d = to_device(case)
    meta = metadata(case, num_parts=num_parts)
    out, lse = run_gpu(d, meta)
    O, LSE = to_np(out, lse)
    O_ref, LSE_ref = run_oracle(case, heads=heads, batches=batches)
    compare(O, LSE, O_ref, LSE_ref, what or case.get("name", ""))
    return meta, out, lse


# ---------------------------------------------------------------- small, full compare

def test_tiny_workload():
    case = make_config(1)
    for P in (0, 1, 3):
        _check(case, num_parts=P, what=f"tiny P={P}")


@pytest.mark.parametrize("s_q,causal,h_q,d_qk", [
    (1, False, 16, 576), (1, False, 128, 576), (2, True, 64, 576), (3, True, 16, 576),
    (1, False, 24, 576), (2, False, 8, 512), (1, False, 128, 512),
    # units of at most 16 rows (the narrow kernel): 16 rows with causal
    # masking, 12 rows of 3 query tokens x 4 heads, a single row
    (2, True, 8, 576), (3, True, 4, 576), (1, False, 1, 512),
    # units of 96, 80 and 160 rows: 128-row workgroups with wavefronts whose
    # 32 rows are all past the unit's, through segment changes (P = 1 walks
    # every request in one part)
    (3, True, 32, 576), (1, False, 80, 576), (5, True, 32, 576),
])
def test_dense_ragged_multi_tile(s_q, causal, h_q, d_qk):
    lens = [1, 63, 64, 65, 700, 2, 130]
    case = make_dense_case(7, B=len(lens), s_q=s_q, h_q=h_q, seqlens=lens, d_qk=d_qk, causal=causal,
                           spare_frac=0.2)
    for P in (0, 1, 5, 37):
        _check(case, num_parts=P, what=f"ragged s_q={s_q} causal={causal} h_q={h_q} d={d_qk} P={P}")


@pytest.mark.parametrize("h_q", [16, 8])
def test_empty_and_fully_masked_rows(h_q):
    # L = 0 (empty request), L = 1 with s_q = 2 causal (query 0 sees nothing),
    # L = 65 with s_q = 2 causal (query 0's last tile is fully masked when split);
    # h_q = 8 gives units of 16 rows (the narrow kernel)
    case = make_dense_case(9, B=4, s_q=2, h_q=h_q, seqlens=[0, 1, 65, 129], causal=True,
                           spare_frac=0.5)
    for P in (0, 1, 3, 9):
        _check(case, num_parts=P, what=f"empty/masked P={P}")


@pytest.mark.parametrize("s_q,active,h_q,d_qk,topk,invalid", [
    (1, 16, 64, 512, 2048, 102), (2, 16, 64, 512, 300, 7), (1, 64, 64, 512, 130, 0),
    (1, 8, 16, 576, 200, 13), (3, 16, 32, 576, 64, 64), (1, 128, 128, 576, 300, 7),
    (2, 96, 128, 512, 520, 33),
])
def test_sparse_small(s_q, active, h_q, d_qk, topk, invalid):
    case = make_sparse_case(13, B=3, s_q=s_q, h_q=h_q, active_h_q=active, topk=topk,
                            cache_len=4096, invalid_tail=invalid, d_qk=d_qk, d_v=512)
    for P in (0, 1, 7):
        _check(case, num_parts=P, what=f"sparse s_q={s_q} act={active} topk={topk} inv={invalid} P={P}")


def test_sparse_invalid_and_duplicate_indices():
    case = make_sparse_case(17, B=2, s_q=1, h_q=16, active_h_q=16, topk=256, cache_len=1024,
                            invalid_tail=0, d_qk=512, d_v=512)
    idx = case["indices"].clone()
    nrows = case["kvcache"].shape[0] * 64
    idx[0, 0, 10:20] = -1
    idx[0, 0, 20:25] = nrows          # out of range: invalid
    idx[0, 0, 25:30] = -12345
    idx[1, 0, 0:40] = idx[1, 0, 40:80]  # duplicates count with multiplicity
    idx[1, 0, 200:256] = -1             # whole last chunk invalid except 8
    case["indices"] = idx
    for P in (0, 1, 3):
        _check(case, num_parts=P, what=f"sparse invalid/dup P={P}")


# ---------------------------------------------------------------- invariants on the GPU

def test_split_count_independence():
    case = make_dense_case(19, B=3, s_q=1, h_q=64, seqlens=[5000, 64, 3000], spare_frac=0.1)
    outs = []
    for P in (1, 7, 64, 256, 1024):
        meta, out, lse = _check(case, num_parts=P, what=f"splits P={P}")
        outs.append((meta.max_splits, out.float().cpu(), lse.cpu()))
    assert max(o[0] for o in outs) > 64  # the combine's multi-pass path ran
    base = outs[0]
    for ms, o, l in outs[1:]:
        # same result up to fp32 reassociation of the split merge
        assert (o - base[1]).abs().max().item() < 2e-2
        assert (l - base[2]).abs().max().item() < 1e-4


def test_run_to_run_bit_identical():
    case = make_dense_case(23, B=4, s_q=2, h_q=128, seqlens=[4000, 100, 2500, 64], causal=True)
    d = to_device(case)
    meta = metadata(case, num_parts=37)
    o1, l1 = run_gpu(d, meta)
    o2, l2 = run_gpu(d, meta)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_block_permutation_bit_identical():
    case = make_dense_case(29, B=3, s_q=1, h_q=32, seqlens=[900, 300, 1281], spare_frac=0.3)
    d = to_device(case)
    meta = metadata(case, num_parts=11)
    o1, l1 = run_gpu(d, meta)
    pool = case["kvcache"].shape[0]
    perm = torch.randperm(pool, generator=torch.Generator().manual_seed(3))
    kv2 = torch.empty_like(case["kvcache"])
    kv2[perm] = case["kvcache"]
    bt2 = case["block_table"].clone()
    m = bt2 >= 0
    bt2[m] = perm[bt2[m].long()].to(torch.int32)
    d2 = dict(d, kvcache=kv2.cuda(), block_table=bt2.cuda())
    o2, l2 = run_gpu(d2, meta)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_nan_poisoned_tails_and_spare_blocks_do_not_leak():
    case = make_dense_case(31, B=3, s_q=2, h_q=16, seqlens=[70, 129, 1], causal=True, spare_frac=1.0)
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
                kv[blk, L % 64:] = float("nan")  # tail of the last page
    for blk in range(kv.shape[0]):
        if blk not in used:
            kv[blk] = float("nan")               # spare pages
    bt = case["block_table"].clone()
    bt[bt < 0] = 0  # unused entries point at a poisoned page (never read)
    d2 = dict(d, kvcache=kv.cuda(), block_table=bt.cuda())
    o2, l2 = run_gpu(d2, meta)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_sparse_active_heads_match_all_heads():
    """Scheduling only the 16 active heads (units of 16 rows: the narrow kernel,
    16-row MFMA blocks) and scheduling all 64 heads (the pair kernel) give the
    active heads the same result up to fp32 reassociation; both also match the
    oracle."""
    case = make_sparse_case(37, B=4, s_q=1, h_q=64, active_h_q=16, topk=512, cache_len=8192,
                            invalid_tail=25, d_qk=512, d_v=512)
    d = to_device(case)
    for P in (0, 5):
        m16 = metadata(case, num_parts=P, active_h_q=16)
        m64 = metadata(case, num_parts=P, active_h_q=64)
        assert m16.rows == 16 and m64.rows == 64
        o16, l16 = run_gpu(d, m16)
        o64, l64 = run_gpu(d, m64)
        assert (o16[:, :, :16].float() - o64[:, :, :16].float()).abs().max() < 2e-2
        assert (l16[:, :, :16] - l64[:, :, :16]).abs().max() < 1e-4
    _check(case, num_parts=5, what="active heads only")


def test_sparse_poisoned_invalid_rows_do_not_leak():
    case = make_sparse_case(41, B=2, s_q=1, h_q=16, active_h_q=16, topk=256, cache_len=2048,
                            invalid_tail=40, d_qk=512, d_v=512)
    d = to_device(case)
    meta = metadata(case, num_parts=3)
    o1, l1 = run_gpu(d, meta)
    kv = case["kvcache"].clone().view(-1, 512)
    keep = torch.zeros(kv.shape[0], dtype=torch.bool)
    iv = case["indices"].flatten()
    keep[iv[iv >= 0].long()] = True
    kv[~keep] = float("nan")
    d2 = dict(d, kvcache=kv.view_as(case["kvcache"]).cuda())
    o2, l2 = run_gpu(d2, meta)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_stages_compose_to_decode():
    import mla_paged_kv_amd as mla
    case = make_dense_case(43, B=3, s_q=1, h_q=64, seqlens=[3000, 70, 900], spare_frac=0.1)
    d = to_device(case)
    meta = metadata(case, num_parts=9)
    assert meta.num_split_units > 0
    o1, l1 = run_gpu(d, meta)
    out, lse, ws = mla.mla_decode_paged(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"],
                                        512, meta, softmax_scale=case["softmax_scale"], stage="split")
    mla.mla_combine(meta, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, out) and torch.equal(l1, lse)


# ---------------------------------------------------------------- the five workloads at full size

@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_named_workload_full_size(k):
    case = make_config(k)
    log(f"workload {k}: {case['name']}")
    # every request of every workload is checked (workload 3: all 128
    # requests, so every workgroup column of its schedule)
    _check(case, num_parts=0, what=f"workload {k}")


@pytest.mark.parametrize("fp8", [False, True])
def test_sparse_whole_tiles_of_invalid_indices(fp8):
    """Tiles whose 64 indices are all invalid are read as zero rows and fully
    masked: the result equals the oracle's and does not change when every
    row the indices do not select (row 0 included) is NaN-poisoned."""
    d_qk = 576
    case = make_sparse_case(45, B=3, s_q=1, h_q=16, active_h_q=16, topk=320, cache_len=4096,
                            invalid_tail=190, d_qk=d_qk, kv_fp8=fp8)
    idx = case["indices"].clone()
    idx[1, 0, :] = -1  # a query with no valid index at all
    case = dict(case, indices=idx)
    _check(case, num_parts=0, what=f"whole invalid tiles fp8={fp8}")
    d = to_device(case)
    meta = metadata(case, num_parts=2)
    o1, l1 = run_gpu(d, meta)
    row_w = case["kvcache"].shape[-1]
    kv = case["kvcache"].clone().view(-1, row_w)
    keep = torch.zeros(kv.shape[0], dtype=torch.bool)
    iv = idx.flatten()
    keep[iv[iv >= 0].long()] = True
    if fp8:
        kv[~keep] = 0xFF
    else:
        kv[~keep] = float("nan")
    o2, l2 = run_gpu(dict(d, kvcache=kv.view_as(case["kvcache"]).cuda()), meta)
    assert torch.equal(o1[:, :, :16], o2[:, :, :16]) and torch.equal(l1[:, :, :16], l2[:, :, :16])
    assert torch.all(torch.isneginf(l1[1, 0, :16])) and torch.all(o1[1, 0, :16] == 0)
