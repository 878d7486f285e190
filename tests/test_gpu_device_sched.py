"""GPU checks of the device tile scheduler (mla_get_metadata_device).

* Its metadata array is bit-identical to the reference scheduler's (oracle)
  for dense and sparse unit lengths: random, skewed, empty units, exact page
  multiples, one part, more parts than work, the largest unit and part counts
  it accepts, and no unit at all.
* A decode that uses it matches the FP64 oracle (same tolerances as the
  parity tests) and the decode with host-built metadata.
* A HIP graph that captures metadata + decode gives, on every replay with new
  cache lengths written into the same device tensor, the eager result for
  those lengths -- with eager work and synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import mla_paged_kv_amd as mla
from oracle.schedule import ref_num_parts, ref_schedule
from synth.configs import make_dense_case, make_sparse_case, rng_for
from tests._gpu_util import compare, log, metadata, run_gpu, run_oracle, to_device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"libmla: {mla.lib_path()}  device: {torch.cuda.get_device_name(0)}")


def _dense_lens(kind, rng, n):
    if kind == "uniform":
        return rng.integers(0, 9000, n)
    if kind == "skewed":
        lens = rng.integers(1, 600, n)
        lens[rng.integers(0, n, max(1, n // 8))] = rng.integers(20000, 140000)
        return lens
    if kind == "pages":
        return 64 * rng.integers(0, 80, n)
    if kind == "zeros":
        lens = rng.integers(0, 3000, n)
        lens[::3] = 0
        return lens
    raise ValueError(kind)


def _assert_close(o1, l1, o2, l2):
    """Same result up to fp32 reassociation of the split merge; rows that see
    no key are -inf in both LSEs."""
    assert (o1.float() - o2.float()).abs().max().item() < 2e-2
    fin = torch.isfinite(l2)
    assert torch.equal(fin, torch.isfinite(l1))
    if fin.any():
        assert (l1[fin] - l2[fin]).abs().max().item() < 1e-4


def _dev_meta_dense(lens, s_q, h_q, P):
    sl = torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda()
    m = mla.mla_get_metadata_device(sl, s_q, h_q, num_parts=P)
    return m, m.exact()


@pytest.mark.parametrize("kind", ["uniform", "skewed", "pages", "zeros"])
@pytest.mark.parametrize("n,P", [(1, 1), (3, 7), (64, 256), (128, 64), (16, 256), (300, 1),
                                 (257, 1024), (4096, 256), (4096, 1024), (1000, 3)])
def test_device_metadata_bit_exact_dense(kind, n, P):
    rng = rng_for(7000 + 31 * n + P)
    lens = _dense_lens(kind, rng, n)
    s_q, h_q = 1 + n % 2, 64
    log(f"device scheduler dense {kind} units={n} P={P}")
    _, got = _dev_meta_dense(lens, s_q, h_q, P)
    want = ref_schedule(lens.tolist(), P, s_q * h_q)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("B,s_q,topk,active,P", [(32, 1, 2048, 64, 0), (8, 2, 300, 16, 5),
                                                 (128, 4, 64, 128, 1), (1, 1, 1, 8, 9)])
def test_device_metadata_bit_exact_sparse(B, s_q, topk, active, P):
    log(f"device scheduler sparse B={B} s_q={s_q} topk={topk} active={active} P={P}")
    m = mla.mla_get_metadata_device(None, s_q, 128, topk=topk, active_h_q=active, num_parts=P,
                                    batch=B)
    host = mla.mla_get_metadata(np.zeros(B, np.int32), s_q, 128, topk=topk, active_h_q=active,
                                num_parts=P, upload=False)
    want = ref_schedule([topk] * (B * s_q), host.target_parts, active)
    np.testing.assert_array_equal(m.exact(), want)
    np.testing.assert_array_equal(host.meta_host, want)


def test_device_metadata_default_parts_and_no_units():
    sl = torch.as_tensor(np.array([4096] * 16 + [100] * 16, np.int32)).cuda()
    m = mla.mla_get_metadata_device(sl, 1, 64)
    P = ref_num_parts(64, torch.cuda.get_device_properties(0).multi_processor_count)
    np.testing.assert_array_equal(m.exact(), ref_schedule(sl.cpu().tolist(), P, 64))
    e = mla.mla_get_metadata_device(torch.zeros(0, dtype=torch.int32, device="cuda"), 1, 64,
                                    num_parts=8)
    np.testing.assert_array_equal(e.exact(), ref_schedule([], 8, 64))


def test_device_metadata_negative_length_gives_empty_schedule():
    sl = torch.as_tensor(np.array([100, -1, 50], np.int32)).cuda()
    m = mla.mla_get_metadata_device(sl, 1, 16, num_parts=4)
    hdr = m.meta_dev[:16].cpu().numpy()
    assert hdr[0] == 0 and hdr[3] == 0 and hdr[15] == -1
    assert hdr[5] == 3 and hdr[11] == 16  # units and rows stay for the decode kernels


@pytest.mark.parametrize("h_q", [16, 128])  # pair kernel (<= 64 rows), decode kernel (> 64 rows)
def test_device_metadata_negative_length_marks_every_output(h_q):
    """A decode with a schedule the device scheduler rejected writes O = 0 and
    LSE = NaN for every row, not what the buffers held before."""
    case = make_dense_case(503, B=3, s_q=1, h_q=h_q, seqlens=[100, 5, 50])
    d = to_device(case)
    sl = torch.as_tensor(np.array([100, -1, 50], np.int32)).cuda()
    m = mla.mla_get_metadata_device(sl, 1, h_q, num_parts=4)
    log(f"rejected device metadata, h_q={h_q}")
    out = torch.full((3, 1, h_q, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((3, 1, h_q), 7.0, dtype=torch.float32, device="cuda")
    mla.mla_decode_paged(d["q"], d["kvcache"], d["block_table"], d["cache_seqlens"], 512, m,
                         softmax_scale=case["softmax_scale"], out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((out == 0).all()), "every output element is 0"
    assert bool(torch.isnan(lse).all()), "every LSE is NaN"


def test_device_metadata_reuses_buffer_across_calls():
    buf = torch.full((40000,), -7, dtype=torch.int32, device="cuda")
    rng = rng_for(77)
    for n, P in ((500, 200), (20, 7), (1, 1)):
        lens = _dense_lens("uniform", rng, n)
        sl = torch.as_tensor(lens.astype(np.int32)).cuda()
        m = mla.mla_get_metadata_device(sl, 1, 32, num_parts=P, meta_out=buf)
        np.testing.assert_array_equal(m.exact(), ref_schedule(lens.tolist(), P, 32))


# h_q = 8: units of 16 rows (the narrow kernel); 64: 128 rows (the decode kernel)
@pytest.mark.parametrize("P,h_q", [(0, 64), (1, 64), (9, 64), (64, 64), (0, 8), (9, 8)])
def test_decode_with_device_metadata_dense(P, h_q):
    case = make_dense_case(501, B=5, s_q=2, h_q=h_q, seqlens=[3000, 1, 700, 64, 1500], causal=True,
                           spare_frac=0.2)
    d = to_device(case)
    log(f"decode with device metadata, dense P={P} h_q={h_q}")
    md = mla.mla_get_metadata_device(d["cache_seqlens"], 2, h_q, num_parts=P)
    out, lse = run_gpu(d, md)
    O, LSE = to_np(out, lse)
    compare(O, LSE, *run_oracle(case), f"device-meta dense P={P} h_q={h_q}")
    mh = metadata(case, num_parts=P)
    np.testing.assert_array_equal(md.exact(), mh.meta_host)
    oh, lh = run_gpu(d, mh)
    _assert_close(out, lse, oh, lh)


# 32 active heads: the pair kernel; 16: the narrow kernel
@pytest.mark.parametrize("P,active", [(0, 32), (3, 32), (0, 16), (3, 16)])
def test_decode_with_device_metadata_sparse(P, active):
    case = make_sparse_case(503, B=4, s_q=2, h_q=64, active_h_q=active, topk=1024, cache_len=6000,
                            invalid_tail=17)
    d = to_device(case)
    log(f"decode with device metadata, sparse P={P} active={active}")
    md = mla.mla_get_metadata_device(None, 2, 64, topk=1024, active_h_q=active, num_parts=P, batch=4)
    out, lse = run_gpu(d, md)
    O, LSE = to_np(out, lse)
    compare(O, LSE, *run_oracle(case), f"device-meta sparse P={P} active={active}")


def test_graph_captured_step_replays_with_new_lengths():
    """Metadata + decode captured once; lengths change between replays."""
    B, s_q, h_q, P = 6, 2, 64, 40
    max_len = 4000
    base = make_dense_case(601, B=B, s_q=s_q, h_q=h_q, seqlens=[max_len] * B, causal=True)
    d = to_device(base)
    sl = d["cache_seqlens"]
    out = torch.empty((B, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device="cuda")
    meta_buf = torch.empty(int(mla._binding._load().mla_metadata_capacity(B, P)),
                           dtype=torch.int32, device="cuda")
    probe = mla.mla_get_metadata_device(sl, s_q, h_q, num_parts=P, meta_out=meta_buf)
    ws = torch.empty(max(1, probe.workspace_bytes()), dtype=torch.uint8, device="cuda")

    def step():
        m = mla.mla_get_metadata_device(sl, s_q, h_q, num_parts=P, meta_out=meta_buf)
        mla.mla_decode_paged(d["q"], d["kvcache"], d["block_table"], sl, 512, m, causal=True,
                             softmax_scale=base["softmax_scale"], workspace=ws, out=out, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    rng = rng_for(602)
    for r, lens in enumerate([rng.integers(0, max_len + 1, B), np.full(B, max_len),
                              np.array([1, 0, 64, 65, 3999, 2000]), rng.integers(0, 300, B)]):
        lens = lens.astype(np.int32)
        sl.copy_(torch.as_tensor(lens))
        torch.cuda.synchronize()
        log(f"graph replay {r}: lens={lens.tolist()}")
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        # eager reference for the same lengths, host-built metadata, fresh buffers
        case = dict(base, cache_seqlens=torch.as_tensor(lens))
        mh = mla.mla_get_metadata(lens, s_q, h_q, num_parts=P)
        np.testing.assert_array_equal(meta_buf.cpu().numpy()[:mh.total_ints], mh.meta_host)
        eo, el = run_gpu(dict(d, cache_seqlens=sl), mh)
        _assert_close(got_o, got_l, eo, el)
        if r == 0:
            O, LSE = to_np(got_o, got_l)
            compare(O, LSE, *run_oracle(case), "graph replay 0")
