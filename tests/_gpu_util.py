"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI
binding, run the FP64 oracle on the same seeded inputs, compare.

Tolerances: relative L2 error of O <= 1e-2 (checked over every compared
element and, more strictly, per query row), every element of O within 5e-2 of
its row's RMS, and absolute LSE error <= 1e-3; a row that sees no key must give
O == 0 exactly and LSE == -inf on both sides.

The element bound: rounding O to bf16 moves an element by at most 2^-9 of
itself (about 0.002 of the row RMS for elements up to 4 RMS), and rounding the
softmax weights to bf16 adds errors of the same relative size that average
over the keys, so 5e-2 leaves more than tenfold headroom while a wrong column
of a few percent fails it.
"""
import sys

import numpy as np
import torch

import mla_paged_kv_amd as mla
import oracle

O_REL_L2 = 1e-2
O_ELEM_RMS = 5e-2
LSE_ABS = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(case, device="cuda"):
    d = dict(case)
    for k in ("q", "kvcache", "block_table", "cache_seqlens", "indices"):
        if d.get(k) is not None:
            d[k] = d[k].to(device).contiguous()
    return d


def metadata(case, num_parts=0, active_h_q=None):
    if case["sparse"]:
        act = case["active_h_q"] if active_h_q is None else active_h_q
        return mla.mla_get_metadata(case["cache_seqlens"].cpu(), case["s_q"], case["h_q"],
                                    topk=case["topk"], active_h_q=act, num_parts=num_parts)
    act = 0 if active_h_q is None else active_h_q
    return mla.mla_get_metadata(case["cache_seqlens"].cpu(), case["s_q"], case["h_q"],
                                active_h_q=act, num_parts=num_parts)


def run_gpu(dcase, meta):
    """dcase: tensors on the GPU.  Returns (O float64 numpy, LSE float64 numpy)."""
    if dcase["sparse"]:
        out, lse = mla.mla_decode_sparse(dcase["q"], dcase["kvcache"], dcase["indices"],
                                         dcase["d_v"], meta, softmax_scale=dcase["softmax_scale"])
    else:
        out, lse = mla.mla_decode_paged(dcase["q"], dcase["kvcache"], dcase["block_table"],
                                        dcase["cache_seqlens"], dcase["d_v"], meta,
                                        causal=dcase["causal"],
                                        softmax_scale=dcase["softmax_scale"])
    torch.cuda.synchronize()
    return out, lse


def to_np(out, lse):
    # widened by torch: padded heads are never written, and numpy's own cast
    # warns on the signalling NaNs such unwritten memory can hold
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def run_oracle(case, heads=None, batches=None):
    if case["sparse"]:
        if heads is None:
            heads = range(case["active_h_q"])
        return oracle.ref_decode_sparse(case["q"], case["kvcache"], case["indices"], case["d_v"],
                                        case["softmax_scale"], heads=heads, batches=batches)
    return oracle.ref_decode_paged(case["q"], case["kvcache"], case["block_table"],
                                   case["cache_seqlens"], case["d_v"], case["causal"],
                                   case["softmax_scale"], heads=heads, batches=batches)


def compare(O, LSE, O_ref, LSE_ref, what=""):
    """Compare on the entries the oracle computed (non-NaN LSE)."""
    sel = ~np.isnan(LSE_ref)
    assert sel.any(), "nothing to compare"
    o, r = O[sel], O_ref[sel]            # [n_rows, dv]
    l, lr = LSE[sel], LSE_ref[sel]
    empty = np.isneginf(lr)
    assert np.array_equal(np.isneginf(l), empty), f"{what}: -inf LSE pattern differs"
    assert np.all(o[empty] == 0), f"{what}: rows with no visible key must be 0"
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    fin = ~empty
    lerr = float(np.max(np.abs(l[fin] - lr[fin]))) if fin.any() else 0.0
    den = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(o - r)) / den if den > 0 else float(np.linalg.norm(o))
    row_den = np.linalg.norm(r[fin], axis=1)
    row_rel = np.linalg.norm(o[fin] - r[fin], axis=1) / np.maximum(row_den, 1e-30)
    worst = float(row_rel.max()) if fin.any() else 0.0
    # every element within O_ELEM_RMS of its row's RMS: a few wrong columns
    # cannot hide under a 512-wide row's L2 norm
    row_rms = np.sqrt(np.mean(r[fin] ** 2, axis=1))
    elem = float(np.max(np.abs(o[fin] - r[fin]) / np.maximum(row_rms, 1e-30)[:, None])) if fin.any() else 0.0
    log(f"  {what}: rows={int(sel.sum())} rel_l2={rel:.3e} worst_row_rel_l2={worst:.3e} "
        f"max_elem/row_rms={elem:.3e} max_lse_err={lerr:.3e}")
    assert rel <= O_REL_L2, f"{what}: rel L2 {rel}"
    assert worst <= O_REL_L2, f"{what}: worst row rel L2 {worst}"
    assert elem <= O_ELEM_RMS, f"{what}: an element is {elem} of its row's RMS off"
    assert lerr <= LSE_ABS, f"{what}: LSE err {lerr}"
    return rel, worst, lerr
