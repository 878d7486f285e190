"""mla_decode_paged_noalloc -- the allocation-free variant of mla_decode_paged
-- against mla_decode_paged itself, through the C-ABI binding.

The two run the same kernels on the same schedule, so their outputs must be
bit-identical; the second of two calls in a row (smaller, with the static
scratch still holding the first call's partials) is also checked against the
FP64 oracle on sampled requests.  A schedule whose partials exceed the static
array is refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import mla_paged_kv_amd as mla
from synth.configs import make_dense_case
from tests._gpu_util import compare, log, run_oracle, to_device, to_np

pytestmark = pytest.mark.gpu


def _noalloc(d, meta):
    out = torch.full((d["q"].shape[0], d["s_q"], d["h_q"], d["d_v"]), 7.0, dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((d["q"].shape[0], d["s_q"], d["h_q"]), 7.0, dtype=torch.float32, device="cuda")
    mla.mla_decode_paged_noalloc(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"],
                                 d["d_v"], meta, causal=d["causal"],
                                 softmax_scale=d["softmax_scale"], out=out, lse=lse)
    return out, lse


def _with_workspace(d, meta):
    return mla.mla_decode_paged(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"],
                                d["d_v"], meta, causal=d["causal"],
                                softmax_scale=d["softmax_scale"])


def _same(a, b, what):
    assert torch.equal(a[0], b[0]), f"{what}: O differs from mla_decode_paged"
    la, lb = a[1].cpu().numpy(), b[1].cpu().numpy()
    assert np.array_equal(la, lb, equal_nan=True), f"{what}: LSE differs from mla_decode_paged"


# the second call's units: 64 rows (the pair kernel) or 16 (the narrow kernel)
@pytest.mark.parametrize("device_meta,small_h_q", [(False, 64), (True, 64), (False, 16), (True, 16)])
def test_noalloc_matches_decode_paged_twice(device_meta, small_h_q):
    big = make_dense_case(71, B=8, s_q=2, h_q=128, causal=True,
                          seqlens=np.random.default_rng(71).integers(1, 4097, 8).tolist(),
                          table_width=64)
    small = make_dense_case(72, B=3, s_q=1, h_q=small_h_q, seqlens=[1, 333, 700], table_width=16)
    runs = []
    for name, case in (("big", big), ("small", small)):
        d = to_device(case)
        if device_meta:
            meta = mla.mla_get_metadata_device(d["cache_seqlens"], case["s_q"], case["h_q"])
        else:
            meta = mla.mla_get_metadata(case["cache_seqlens"], case["s_q"], case["h_q"])
        need = meta.workspace_bytes(512)
        log(f"case {name}: device_meta={device_meta} workspace {need} bytes")
        assert 0 < need <= (128 << 20)
        runs.append((name, case, d, meta, _noalloc(d, meta)))
    torch.cuda.synchronize()
    assert runs[1][3].workspace_bytes(512) < runs[0][3].workspace_bytes(512)
    for name, case, d, meta, got in runs:
        ref = _with_workspace(d, meta)
        torch.cuda.synchronize()
        _same(got, ref, name)
    # the second (smaller) call, run over the first call's leftovers, against the oracle
    name, case, d, meta, got = runs[1]
    O, L = to_np(*got)
    Or, Lr = run_oracle(case)
    compare(O, L, Or, Lr, f"noalloc {name} vs oracle")


def test_noalloc_refuses_schedules_beyond_the_scratch():
    B, h_q = 4, 128
    lens = torch.full((B,), 65536, dtype=torch.int32)
    meta = mla.mla_get_metadata(lens, 1, h_q, num_parts=1024)
    assert meta.workspace_bytes(512) > (128 << 20)
    q = torch.zeros((B, 1, h_q, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 64, 1, 576), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, 1024), dtype=torch.int32, device="cuda")
    out = torch.full((B, 1, h_q, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, 1, h_q), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_paged_noalloc(q, kv, bt, lens.cuda(), 512, meta, out=out, lse=lse)
    assert "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
