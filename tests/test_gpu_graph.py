"""The decode launches captured in a HIP graph (torch.cuda.CUDAGraph over the
C-ABI calls, as bench.py times them and a serving loop would run them).

The split-KV and combine launches of one decode step are captured once and
replayed several times, with the program's own eager work (other decode
calls, torch ops, output clearing) and synchronisations between replays.
Every replay must reproduce the eager result of the same launches bit for
bit, and that result matches the FP64 oracle.  Dense (split units present)
and sparse (active heads) paths.
"""
import pytest
import torch

import mla_paged_kv_amd as mla
from synth.configs import make_dense_case, make_sparse_case
from tests._gpu_util import compare, log, metadata, run_oracle, to_device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"libmla: {mla.lib_path()}  device: {torch.cuda.get_device_name(0)}")


def _launch(d, meta, out, lse, ws):
    if d["sparse"]:
        mla.mla_decode_sparse(d["q"], d["kvcache"], d["indices"], d["d_v"], meta,
                              softmax_scale=d["softmax_scale"], workspace=ws, out=out, lse=lse,
                              stage="split")
    else:
        mla.mla_decode_paged(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"], d["d_v"],
                             meta, causal=d["causal"], softmax_scale=d["softmax_scale"],
                             workspace=ws, out=out, lse=lse, stage="split")
    mla.mla_combine(meta, out, lse, ws, d["d_v"])


def _buffers(d, meta):
    B, s_q, h_q = d["q"].shape[:3]
    out = torch.empty((B, s_q, h_q, d["d_v"]), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(meta.workspace_bytes(d["d_v"]), 256), dtype=torch.uint8, device="cuda")
    return out, lse, ws


@pytest.mark.parametrize("kind", ["dense", "sparse"])
def test_graph_replays_match_eager(kind):
    if kind == "dense":
        case = make_dense_case(901, B=5, s_q=2, h_q=64, seqlens=[3000, 70, 900, 1, 2500], causal=True)
        other = make_dense_case(902, B=2, s_q=1, h_q=16, seqlens=[300, 40])
    else:
        case = make_sparse_case(903, B=4, s_q=1, h_q=64, active_h_q=16, topk=1024, cache_len=4096,
                                invalid_tail=50, d_qk=576)
        other = make_sparse_case(904, B=2, s_q=1, h_q=16, active_h_q=16, topk=256, cache_len=1024,
                                 invalid_tail=10, d_qk=576)
    d, d2 = to_device(case), to_device(other)
    meta, meta2 = metadata(case, num_parts=11), metadata(other)
    log(f"graph {kind}: split units {meta.num_split_units}")
    if kind == "dense":
        assert meta.num_split_units > 0

    # eager reference of the same launches
    out_e, lse_e, ws_e = _buffers(d, meta)
    _launch(d, meta, out_e, lse_e, ws_e)
    torch.cuda.synchronize()
    compare(*to_np(out_e, lse_e), *run_oracle(case), f"graph {kind} eager")

    out_g, lse_g, ws_g = _buffers(d, meta)
    _launch(d, meta, out_g, lse_g, ws_g)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _launch(d, meta, out_g, lse_g, ws_g)
    torch.cuda.synchronize()

    # sparse calls write the active heads only
    act = slice(None) if kind == "dense" else slice(0, case["active_h_q"])
    o2, l2, w2 = _buffers(d2, meta2)
    for rep in range(4):
        # the program's own eager work between replays
        out_g.fill_(0)
        lse_g.fill_(float("nan"))
        _launch(d2, meta2, o2, l2, w2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"graph {kind}: replay {rep}")
        assert torch.equal(out_g[:, :, act], out_e[:, :, act]), \
            f"replay {rep}: out differs from the eager launches"
        assert torch.equal(lse_g[:, :, act], lse_e[:, :, act]), \
            f"replay {rep}: lse differs from the eager launches"
    del g
