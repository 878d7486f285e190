"""GPU parity of sparse MLA prefill (mla_sparse_prefill / flash_mla_sparse_fwd)
against the FP64 oracle of the page's equations (out, max_logits, base-2 lse).

Small cases are compared on every output: ragged index lists with both kinds of
invalid entries (-1 and >= s_kv), s_kv not a multiple of 64, d_qk 576 and 512,
head counts from 16 to 128, forced split counts (the combine then merges the
partial maxima too), all-invalid query tokens.  The 4096-token chunk over a
32768-token context runs at full size in the benchmark's launch configuration
and is compared on sampled query tokens.
"""
import numpy as np
import pytest
import torch

import mla_paged_kv_amd as mla
from oracle import ref_sparse_prefill
from synth.configs import make_config, make_prefill_case
from tests._gpu_util import LSE_ABS, O_REL_L2, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"libmla: {mla.lib_path()}  device: {torch.cuda.get_device_name(0)}")


def _run(case, num_parts=0):
    q, kv, idx = case["q"].cuda(), case["kv"].cuda(), case["indices"].cuda()
    meta = None
    if num_parts:
        meta = mla.mla_get_metadata(np.zeros(case["s_q"], np.int32), 1, case["h_q"],
                                    topk=case["topk"], num_parts=num_parts)
    out, mx, lse = mla.mla_sparse_prefill(q, kv, idx, case["softmax_scale"], dv=case["d_v"],
                                          meta=meta)
    torch.cuda.synchronize()
    return (out.double().cpu().numpy(), mx.double().cpu().numpy(),
            lse.double().cpu().numpy())


def _compare(got, ref, rows, what):
    O, M, L = got
    Or, Mr, Lr = ref
    O, M, L, Or, Mr, Lr = (a[rows] for a in (O, M, L, Or, Mr, Lr))
    empty = np.isneginf(Lr)
    assert np.array_equal(np.isneginf(L), empty) and np.array_equal(np.isneginf(M), empty), what
    assert np.all(O[empty] == 0), what
    fin = ~empty
    rel = np.linalg.norm(O - Or) / max(np.linalg.norm(Or), 1e-30)
    lerr = float(np.abs(L[fin] - Lr[fin]).max()) if fin.any() else 0.0
    merr = float(np.abs(M[fin] - Mr[fin]).max()) if fin.any() else 0.0
    # base-2 quantities: |d lse2| <= 1e-3 / ln 2 is the natural-log bound
    log(f"  {what}: rel_l2={rel:.3e} max_lse2_err={lerr:.3e} max_logit_err={merr:.3e}")
    assert rel <= O_REL_L2, what
    assert lerr <= LSE_ABS / np.log(2), what
    assert merr <= LSE_ABS / np.log(2), what


@pytest.mark.parametrize("h_q,d_qk,topk,P", [(16, 576, 300, 0), (64, 576, 700, 7), (128, 576, 2048, 0),
                                            (128, 512, 256, 1), (32, 576, 130, 40)])
def test_prefill_small(h_q, d_qk, topk, P):
    case = make_prefill_case(901, s_q=37, s_kv=2500, h_q=h_q, topk=topk, d_qk=d_qk,
                             invalid_tail=topk // 10, past_end=topk // 20)
    log(f"prefill h_q={h_q} d_qk={d_qk} topk={topk} P={P}")
    got = _run(case, num_parts=P)
    ref = ref_sparse_prefill(case["q"], case["kv"], case["indices"], case["softmax_scale"], case["d_v"])
    _compare(got, ref, slice(None), f"prefill h_q={h_q} d_qk={d_qk} topk={topk} P={P}")


def test_prefill_all_invalid_queries_and_pages_call():
    case = make_prefill_case(903, s_q=9, s_kv=130, h_q=16, topk=64)
    idx = case["indices"].clone()
    idx[2] = -1
    idx[5] = 130 + torch.arange(64, dtype=torch.int32)  # all past the end
    case = dict(case, indices=idx)
    out, mx, lse = mla.flash_mla_sparse_fwd(case["q"].cuda(), case["kv"].cuda(), idx.cuda(),
                                            case["softmax_scale"])
    torch.cuda.synchronize()
    got = (out.double().cpu().numpy(), mx.double().cpu().numpy(),
           lse.double().cpu().numpy())
    ref = ref_sparse_prefill(case["q"], case["kv"], idx, case["softmax_scale"])
    _compare(got, ref, slice(None), "all-invalid rows")
    assert np.all(np.isneginf(got[2][[2, 5]]))


def test_prefill_chunk_full_size():
    case = make_config("p")
    log(f"workload: {case['name']}")
    got = _run(case)
    rows = list(range(0, case["s_q"], 257)) + [case["s_q"] - 1]
    ref = ref_sparse_prefill(case["q"], case["kv"], case["indices"], case["softmax_scale"],
                             case["d_v"], rows=rows)
    _compare(got, ref, rows, "prefill chunk (sampled)")
