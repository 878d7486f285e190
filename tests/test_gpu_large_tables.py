"""GPU parity with block tables and index lists past byte 2^32.

A unit of more than 64 query rows normally runs on the decode kernel, which
reads the block table (dense) or the index lists (sparse) with 32-bit byte
offsets below 2^31; a larger table goes to the pair kernel, which addresses
it with 64-bit pointers.  Each call here has a table of more than 4 GiB and
128 query heads; the sampled requests (or query tokens) start before 2^31,
between 2^31 and 2^32, and past 2^32 bytes into the table, and are checked
against the FP64 oracle with the tolerances of the other parity tests.
"""
import numpy as np
import pytest
import torch

import mla_paged_kv_amd as mla
import oracle
from synth.configs import make_dense_case
from tests._gpu_util import compare, log, to_device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"libmla: {mla.lib_path()}  device: {torch.cuda.get_device_name(0)}")


def test_dense_block_table_past_4gib():
    B, width = 520, 2 ** 21 + 64  # 4.36e9 bytes; rows from 512 on start past 2^32
    rng = np.random.default_rng(4242)
    seqlens = rng.integers(1, 300, size=B)
    case = make_dense_case(4243, B=B, s_q=1, h_q=128, seqlens=seqlens, d_qk=576, d_v=512)
    small = case["block_table"]
    log(f"dense: B={B}, block table {B} x {width} ({B * width * 4 / 2**30:.2f} GiB)")
    d = to_device(case)
    big = torch.zeros((B, width), dtype=torch.int32, device="cuda")
    big[:, :small.shape[1]] = d["block_table"]
    meta = mla.mla_get_metadata(case["cache_seqlens"], 1, 128)
    out, lse = mla.mla_decode_paged(d["q"], d["kvcache"], big, d["cache_seqlens"], 512, meta,
                                    causal=False, softmax_scale=case["softmax_scale"])
    torch.cuda.synchronize()
    O, LSE = to_np(out, lse)
    del big, d
    torch.cuda.empty_cache()
    batches = [0, 255, 256, 400, 511, 512, 519]
    O_ref, LSE_ref = oracle.ref_decode_paged(case["q"], case["kvcache"], small,
                                             case["cache_seqlens"], 512, False,
                                             case["softmax_scale"], batches=batches)
    compare(O, LSE, O_ref, LSE_ref, "dense block table past 4 GiB")


def test_sparse_index_lists_past_4gib():
    B, topk, pool_rows = 4100, 2 ** 18, 65536  # 4.30e9 bytes of indices
    g = torch.Generator(device="cuda")
    g.manual_seed(4244)
    log(f"sparse: {B} query tokens x top-{topk} ({B * topk * 4 / 2**30:.2f} GiB of indices)")
    q = torch.randn((B, 1, 128, 576), generator=g, device="cuda").to(torch.bfloat16)
    kv = torch.randn((pool_rows // 64, 64, 1, 576), generator=g, device="cuda").to(torch.bfloat16)
    # about 0.1 % of the entries invalid (-1)
    idx = torch.randint(-64, pool_rows, (B, 1, topk), generator=g, device="cuda",
                        dtype=torch.int32).clamp_(min=-1)
    meta = mla.mla_get_metadata(torch.full((B,), pool_rows, dtype=torch.int32), 1, 128,
                                topk=topk, active_h_q=128)
    scale = 576 ** -0.5
    out, lse = mla.mla_decode_sparse(q, kv, idx, 512, meta, softmax_scale=scale)
    torch.cuda.synchronize()
    # tokens 2048.. start past 2^31 bytes of indices, 4096.. past 2^32
    sel = [0, 2047, 2048, 4095, 4096, 4099]
    O = out[sel].double().cpu().numpy()
    LSE = lse[sel].double().cpu().numpy()
    q_s, idx_s, kv_c = q[sel].cpu(), idx[sel].cpu(), kv.cpu()
    del q, kv, idx, out, lse
    torch.cuda.empty_cache()
    O_ref, LSE_ref = oracle.ref_decode_sparse(q_s, kv_c, idx_s, 512, scale)
    compare(O, LSE, O_ref, LSE_ref, "sparse index lists past 4 GiB")
