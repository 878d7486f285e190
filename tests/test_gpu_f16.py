"""GPU parity of the fp16 path (q, cache and output in IEEE fp16) against the
FP64 oracle: dense ragged multi-tile decode (causal and not, forced split
counts, d_qk 576 and 512), sparse decode with active heads, the split-KV +
combine stages, sparse prefill, and the varlen workload's shape at full size
(sampled requests).  Same tolerances as the bf16 tests; fp16 keeps 3 more
mantissa bits, so the errors are smaller.
"""
import numpy as np
import pytest
import torch

import mla_paged_kv_amd as mla
from oracle import ref_sparse_prefill
from synth.configs import _c2_lens, make_dense_case, make_prefill_case, make_sparse_case
from tests._gpu_util import compare, log, metadata, run_gpu, run_oracle, to_device, to_np

pytestmark = pytest.mark.gpu
F16 = torch.float16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"libmla: {mla.lib_path()}  device: {torch.cuda.get_device_name(0)}")


def _check(case, num_parts=0, batches=None, what=""):
    log(f"case {what}: num_parts={num_parts}")
    d = to_device(case)
    meta = metadata(case, num_parts=num_parts)
    out, lse = run_gpu(d, meta)
    assert out.dtype == F16
    O, LSE = to_np(out, lse)
    compare(O, LSE, *run_oracle(case, batches=batches), what)
    return meta, out, lse


@pytest.mark.parametrize("s_q,causal,h_q,d_qk", [(1, False, 16, 576), (2, True, 64, 576),
                                                 (1, False, 128, 512), (3, True, 8, 576)])
def test_f16_dense_ragged(s_q, causal, h_q, d_qk):
    lens = [1, 63, 64, 65, 700, 2, 130]
    case = make_dense_case(701, B=len(lens), s_q=s_q, h_q=h_q, seqlens=lens, d_qk=d_qk,
                           causal=causal, spare_frac=0.2, dtype=F16)
    for P in (0, 1, 5, 37):
        _check(case, num_parts=P, what=f"f16 ragged s_q={s_q} causal={causal} h_q={h_q} d={d_qk} P={P}")


@pytest.mark.parametrize("active,P", [(16, 0), (64, 5)])
def test_f16_sparse(active, P):
    case = make_sparse_case(703, B=4, s_q=2, h_q=64, active_h_q=active, topk=1024,
                            cache_len=6000, invalid_tail=37, d_qk=576, dtype=F16)
    _check(case, num_parts=P, what=f"f16 sparse active={active} P={P}")


def test_f16_stages_compose_to_decode():
    case = make_dense_case(705, B=3, s_q=1, h_q=64, seqlens=[3000, 70, 900], dtype=F16)
    d = to_device(case)
    meta = metadata(case, num_parts=9)
    assert meta.num_split_units > 0
    o1, l1 = run_gpu(d, meta)
    out, lse, ws = mla.mla_decode_paged(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"],
                                        512, meta, softmax_scale=case["softmax_scale"], stage="split")
    mla.mla_combine(meta, out, lse, ws)
    torch.cuda.synchronize()
    assert out.dtype == F16 and torch.equal(o1, out) and torch.equal(l1, lse)


def test_f16_sparse_prefill():
    case = make_prefill_case(707, s_q=29, s_kv=3000, h_q=128, topk=600, invalid_tail=40,
                             past_end=20, dtype=F16)
    out, mx, lse = mla.flash_mla_sparse_fwd(case["q"].cuda(), case["kv"].cuda(),
                                            case["indices"].cuda(), case["softmax_scale"])
    torch.cuda.synchronize()
    assert out.dtype == F16
    Or, Mr, Lr = ref_sparse_prefill(case["q"], case["kv"], case["indices"], case["softmax_scale"])
    O = out.double().cpu().numpy()
    rel = np.linalg.norm(O - Or) / np.linalg.norm(Or)
    lerr = np.abs(lse.cpu().numpy() - Lr).max()
    merr = np.abs(mx.cpu().numpy() - Mr).max()
    log(f"  f16 prefill: rel_l2={rel:.3e} lse2_err={lerr:.3e} max_logit_err={merr:.3e}")
    assert rel <= 1e-2 and lerr <= 1e-3 / np.log(2) and merr <= 1e-3 / np.log(2)


def test_f16_varlen_full_size():
    case = make_dense_case(1002, B=64, s_q=1, h_q=128, seqlen_sampler=_c2_lens, spare_frac=0.1,
                           table_width=64, dtype=F16)
    _check(case, num_parts=0, batches=list(range(0, 64, 7)), what="f16 varlen B=64 h_q=128")


def test_mixed_dtypes_rejected():
    case = make_dense_case(709, B=1, s_q=1, h_q=16, seqlens=[100])
    d = to_device(case)
    meta = metadata(case)
    with pytest.raises(ValueError):
        mla.mla_decode_paged(d["q"].to(F16), d["kvcache"], d["block_table"], d["cache_seqlens"],
                             512, meta)
