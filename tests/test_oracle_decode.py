"""Pins for the FP64 decode oracle, independent of the oracle itself.

Each test checks ``oracle.ref_decode_paged`` / ``ref_decode_sparse`` against
something other than the oracle: a library attention routine (torch's CPU
flash-attention op, float64, which also returns the log-sum-exp), a pure-Python
brute force, closed forms, and invariants the definition implies.  A final
group plants plausible mistakes into the oracle and checks that the pins catch
every one of them.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import decode as odec
from synth.configs import make_config, make_dense_case, make_sparse_case, normal_bf16, rng_for
from tests._brute import brute_paged, brute_sparse

TOL = 1e-12


def _lib_attention(q, k, dv, scale, mask=None):
    """torch CPU flash attention in float64: q [H, m, d], k [H, n, d].

    The op wants equal head sizes, so it runs with value = the whole key row
    and the first ``dv`` output columns are kept (the value is the first ``dv``
    columns of each row)."""
    out, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        q[None].contiguous(), k[None].contiguous(), k[None].contiguous(), 0.0, False,
        attn_mask=mask, scale=scale)
    return out[0, ..., :dv].numpy(), lse[0].numpy()


def _contiguous_case(seed, B, s_q, h_q, d_qk, d_v, lens, h_kv=1):
    """Identity block table: request b's blocks are physical blocks in order."""
    rng = rng_for(seed)
    nb = [(L + 63) // 64 for L in lens]
    width = max(1, max(nb))
    table = np.full((B, width), -1, dtype=np.int32)
    cur = 0
    for b, n in enumerate(nb):
        table[b, :n] = np.arange(cur, cur + n)
        cur += n
    q = normal_bf16(rng, (B, s_q, h_q, d_qk))
    kv = normal_bf16(rng, (max(1, cur), 64, h_kv, d_qk))
    return q, kv, torch.from_numpy(table), torch.tensor(lens, dtype=torch.int32)


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("d_qk,d_v,h_q,lens", [
    (576, 512, 16, [64, 200, 1]),
    (512, 512, 8, [130, 7]),
    (576, 512, 4, [4096]),
])
def test_matches_library_attention_identity_table(d_qk, d_v, h_q, lens):
    B = len(lens)
    q, kv, bt, sl = _contiguous_case(7, B, 1, h_q, d_qk, d_v, lens)
    scale = d_qk ** -0.5
    O, LSE = oracle.ref_decode_paged(q, kv, bt, sl, d_v, False, scale)
    kv64 = kv.to(torch.float64)[:, :, 0, :].reshape(-1, d_qk)
    start = 0
    for b, L in enumerate(lens):
        nb = (L + 63) // 64
        K = kv64[start * 64:start * 64 + L]
        start += nb
        qb = q[b, 0].to(torch.float64)  # [h_q, d]
        o, lse = _lib_attention(qb[:, None, :], K[None].expand(h_q, -1, -1), d_v, scale)
        np.testing.assert_allclose(O[b, 0], o[:, 0, :], rtol=0, atol=TOL)
        np.testing.assert_allclose(LSE[b, 0], lse[:, 0], rtol=0, atol=TOL)


def test_matches_library_attention_causal_mtp():
    s_q, h_q, d_qk, d_v, L = 3, 4, 576, 512, 150
    q, kv, bt, sl = _contiguous_case(11, 1, s_q, h_q, d_qk, d_v, [L])
    scale = d_qk ** -0.5
    O, LSE = oracle.ref_decode_paged(q, kv, bt, sl, d_v, True, scale)
    K = kv.to(torch.float64)[:, :, 0, :].reshape(-1, d_qk)[:L]
    # bottom-right causal mask: query i sees positions <= L - s_q + i
    mask = torch.zeros(s_q, L, dtype=torch.float64)
    for i in range(s_q):
        mask[i, L - s_q + i + 1:] = -math.inf
    qh = q[0].to(torch.float64).permute(1, 0, 2)  # [h_q, s_q, d]
    o, lse = _lib_attention(qh, K[None].expand(h_q, -1, -1), d_v, scale, mask)
    np.testing.assert_allclose(O[0], o.transpose(1, 0, 2), rtol=0, atol=TOL)
    np.testing.assert_allclose(LSE[0], lse.T, rtol=0, atol=TOL)


# ---------------------------------------------------------------- brute force

def _check_brute(O, LSE, ref):
    for (b, i, h), (o, lse) in ref.items():
        np.testing.assert_allclose(O[b, i, h], o, rtol=0, atol=1e-11)
        if math.isinf(lse):
            assert math.isinf(LSE[b, i, h]) and LSE[b, i, h] < 0
        else:
            assert abs(LSE[b, i, h] - lse) < 1e-11


def test_brute_force_tiny_config():
    c = make_config(1)
    O, LSE = oracle.ref_decode_paged(c["q"], c["kvcache"], c["block_table"], c["cache_seqlens"],
                                     c["d_v"], c["causal"], c["softmax_scale"])
    heads = [0, 5, 15]
    ref = brute_paged(c["q"], c["kvcache"], c["block_table"], c["cache_seqlens"], c["d_v"],
                      c["causal"], c["softmax_scale"], heads=heads)
    _check_brute(O, LSE, ref)


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 10_000), B=st.integers(1, 3), s_q=st.integers(1, 3),
       h_kv=st.sampled_from([1, 2]), group=st.integers(1, 2), causal=st.booleans(),
       lens=st.lists(st.integers(0, 200), min_size=3, max_size=3))
def test_brute_force_random_small(seed, B, s_q, h_kv, group, causal, lens):
    h_q = h_kv * group
    d_qk, d_v = 24, 16
    case = make_dense_case(seed, B=B, s_q=s_q, h_q=h_q, seqlens=lens[:B], d_qk=d_qk, d_v=d_v,
                           h_kv=h_kv, causal=causal, spare_frac=0.5)
    O, LSE = oracle.ref_decode_paged(case["q"], case["kvcache"], case["block_table"],
                                     case["cache_seqlens"], d_v, causal, 0.37)
    ref = brute_paged(case["q"], case["kvcache"], case["block_table"], case["cache_seqlens"],
                      d_v, causal, 0.37)
    _check_brute(O, LSE, ref)


@settings(max_examples=20, deadline=None)
@given(seed=st.integers(0, 10_000), topk=st.integers(1, 150), invalid=st.integers(0, 20),
       s_q=st.integers(1, 2))
def test_brute_force_sparse_random_small(seed, topk, invalid, s_q):
    invalid = min(invalid, topk)
    case = make_sparse_case(seed, B=2, s_q=s_q, h_q=4, active_h_q=4, topk=topk,
                            cache_len=200, invalid_tail=invalid, d_qk=24, d_v=24)
    O, LSE = oracle.ref_decode_sparse(case["q"], case["kvcache"], case["indices"], 24, 0.41)
    ref = brute_sparse(case["q"], case["kvcache"], case["indices"], 24, 0.41)
    _check_brute(O, LSE, ref)


# ---------------------------------------------------------------- closed forms

def _small_dense(seed=3, L=100, h_q=4, d_qk=32, d_v=16, s_q=1):
    return make_dense_case(seed, B=1, s_q=s_q, h_q=h_q, seqlens=[L], d_qk=d_qk, d_v=d_v,
                           spare_frac=1.0)


def test_single_token_cache_gives_that_value_row():
    c = _small_dense(L=1)
    O, LSE = oracle.ref_decode_paged(c["q"], c["kvcache"], c["block_table"], c["cache_seqlens"],
                                     16, False, 0.5)
    blk = int(c["block_table"][0, 0])
    row = c["kvcache"][blk, 0, 0].to(torch.float64).numpy()
    qd = c["q"][0, 0].to(torch.float64).numpy()
    for h in range(4):
        np.testing.assert_array_equal(O[0, 0, h], row[:16])
        assert abs(LSE[0, 0, h] - 0.5 * float(np.dot(qd[h], row))) < 1e-12


def test_constant_value_rows_give_that_row():
    c = _small_dense(L=150)
    kv = c["kvcache"].clone()
    const = torch.linspace(-2, 2, 16).to(torch.bfloat16)
    kv[:, :, 0, :16] = const  # every V part equal; keys (all 32 columns) still differ in 16..31
    O, _ = oracle.ref_decode_paged(c["q"], kv, c["block_table"], c["cache_seqlens"], 16, False, 0.3)
    for h in range(4):
        np.testing.assert_allclose(O[0, 0, h], const.to(torch.float64).numpy(), rtol=0, atol=1e-12)


def test_zero_query_gives_mean_of_values_and_log_n():
    c = _small_dense(L=77)
    q = torch.zeros_like(c["q"])
    O, LSE = oracle.ref_decode_paged(q, c["kvcache"], c["block_table"], c["cache_seqlens"], 16, False, 1.0)
    rows = []
    for t in range(77):
        rows.append(c["kvcache"][int(c["block_table"][0, t // 64]), t % 64, 0, :16].to(torch.float64).numpy())
    mean = np.mean(np.stack(rows), axis=0)
    for h in range(4):
        np.testing.assert_allclose(O[0, 0, h], mean, rtol=0, atol=1e-12)
        assert abs(LSE[0, 0, h] - math.log(77)) < 1e-12


def test_empty_cache_gives_zero_and_minus_inf():
    c = make_dense_case(5, B=2, s_q=2, h_q=2, seqlens=[0, 1], d_qk=16, d_v=8, causal=True)
    O, LSE = oracle.ref_decode_paged(c["q"], c["kvcache"], c["block_table"], c["cache_seqlens"], 8, True, 0.2)
    assert np.all(O[0] == 0) and np.all(np.isneginf(LSE[0]))
    # request 1 has L=1, s_q=2: query 0 sees L - 2 + 0 + 1 = 0 positions, query 1 sees 1
    assert np.all(O[1, 0] == 0) and np.all(np.isneginf(LSE[1, 0]))
    assert np.all(np.isfinite(LSE[1, 1]))


# ---------------------------------------------------------------- invariants

def test_block_permutation_invariance():
    c = make_dense_case(21, B=3, s_q=1, h_q=4, seqlens=[300, 64, 129], d_qk=32, d_v=16, spare_frac=0.3)
    O1, L1 = oracle.ref_decode_paged(c["q"], c["kvcache"], c["block_table"], c["cache_seqlens"], 16, False, 0.3)
    pool = c["kvcache"].shape[0]
    perm = torch.randperm(pool, generator=torch.Generator().manual_seed(4))
    kv2 = torch.empty_like(c["kvcache"])
    kv2[perm] = c["kvcache"]  # block p moves to perm[p]
    bt2 = c["block_table"].clone()
    valid = bt2 >= 0
    bt2[valid] = perm[bt2[valid].long()].to(torch.int32)
    O2, L2 = oracle.ref_decode_paged(c["q"], kv2, bt2, c["cache_seqlens"], 16, False, 0.3)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def test_causal_row_equals_shorter_noncausal_call():
    s_q, L = 3, 200
    c = make_dense_case(31, B=1, s_q=s_q, h_q=4, seqlens=[L], d_qk=32, d_v=16)
    O, LSE = oracle.ref_decode_paged(c["q"], c["kvcache"], c["block_table"], c["cache_seqlens"], 16, True, 0.3)
    for i in range(s_q):
        sl = torch.tensor([L - s_q + i + 1], dtype=torch.int32)
        o, lse = oracle.ref_decode_paged(c["q"][:, i:i + 1], c["kvcache"], c["block_table"], sl, 16, False, 0.3)
        np.testing.assert_allclose(O[:, i], o[:, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(LSE[:, i], lse[:, 0], rtol=0, atol=1e-13)


def _merge(parts):
    """Merge per-chunk (O_c, LSE_c) by their log-sum-exp weights."""
    lses = np.array([p[1] for p in parts])
    top = lses.max()
    lse = top + math.log(sum(math.exp(x - top) for x in lses))
    o = sum(math.exp(p[1] - lse) * p[0] for p in parts)
    return o, lse


def test_chunked_merge_equals_unsplit():
    c = _small_dense(seed=8, L=250, h_q=2)
    sl = c["cache_seqlens"]
    q = c["q"][0, 0].to(torch.float64).numpy()
    rows = np.stack([c["kvcache"][int(c["block_table"][0, t // 64]), t % 64, 0].to(torch.float64).numpy()
                     for t in range(250)])
    O, LSE = oracle.ref_decode_paged(c["q"], c["kvcache"], c["block_table"], sl, 16, False, 0.3)
    for cuts in ([0, 64, 128, 192, 250], [0, 1, 249, 250], [0, 100, 250]):
        parts = [odec.ref_attend_rows(q, rows[a:b], 16, 0.3) for a, b in zip(cuts[:-1], cuts[1:])]
        for h in range(2):
            o, lse = _merge([(p[0][h], p[1][h]) for p in parts])
            np.testing.assert_allclose(O[0, 0, h], o, rtol=0, atol=1e-12)
            assert abs(LSE[0, 0, h] - lse) < 1e-12


def test_sparse_all_positions_equals_dense():
    c = make_dense_case(41, B=2, s_q=1, h_q=4, seqlens=[190, 64], d_qk=32, d_v=32, spare_frac=0.5)
    O, LSE = oracle.ref_decode_paged(c["q"], c["kvcache"], c["block_table"], c["cache_seqlens"], 32, False, 0.25)
    idx = torch.full((2, 1, 200), -1, dtype=torch.int32)
    for b, L in enumerate([190, 64]):
        pos = torch.arange(L)
        idx[b, 0, :L] = c["block_table"][b, pos // 64] * 64 + pos % 64
    # scramble order: the set, not the order, defines the result
    idx = idx[:, :, torch.randperm(200, generator=torch.Generator().manual_seed(1))]
    O2, LSE2 = oracle.ref_decode_sparse(c["q"], c["kvcache"], idx, 32, 0.25)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE2, LSE, rtol=0, atol=1e-12)


def test_sparse_invalid_entries_are_removed():
    c = make_sparse_case(51, B=1, s_q=1, h_q=2, active_h_q=2, topk=40, cache_len=256,
                         invalid_tail=0, d_qk=32, d_v=32)
    idx = c["indices"]
    O, LSE = oracle.ref_decode_sparse(c["q"], c["kvcache"], idx[:, :, :30], 32, 0.3)
    nb = c["kvcache"].shape[0]
    bad = idx.clone()
    bad[:, :, 30:35] = -1
    bad[:, :, 35:38] = nb * 64
    bad[:, :, 38:40] = -7
    O2, LSE2 = oracle.ref_decode_sparse(c["q"], c["kvcache"], bad, 32, 0.3)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, LSE2)


def test_sparse_matches_base2_prefill_equations():
    """The sparse-prefill listing works in base 2 with scores pre-multiplied by
    log2(e); its weights are the same, and its lse is the natural LSE / ln 2."""
    c = make_sparse_case(61, B=1, s_q=1, h_q=3, active_h_q=3, topk=50, cache_len=128,
                         invalid_tail=5, d_qk=32, d_v=32)
    scale = 0.3
    O, LSE = oracle.ref_decode_sparse(c["q"], c["kvcache"], c["indices"], 32, scale)
    flat = c["kvcache"].to(torch.float64).reshape(-1, 1, 32)[:, 0]
    sel = c["indices"][0, 0]
    sel = sel[sel >= 0].long()
    focused = flat[sel]
    Q = c["q"][0, 0].to(torch.float64)
    P = (Q @ focused.T) * scale * math.log2(math.e)
    lse2 = torch.log2(torch.exp2(P - P.max(-1, keepdim=True).values).sum(-1)) + P.max(-1).values
    out = torch.exp2(P - lse2[:, None]) @ focused
    np.testing.assert_allclose(O[0, 0], out.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE[0, 0], (lse2 * math.log(2)).numpy(), rtol=0, atol=1e-12)


def test_head_subset_matches_full():
    c = make_sparse_case(71, B=2, s_q=1, h_q=8, active_h_q=2, topk=64, cache_len=256,
                         invalid_tail=3, d_qk=32, d_v=32)
    Of, Lf = oracle.ref_decode_sparse(c["q"], c["kvcache"], c["indices"], 32, 0.3)
    Os, Ls = oracle.ref_decode_sparse(c["q"], c["kvcache"], c["indices"], 32, 0.3, heads=range(2))
    np.testing.assert_array_equal(Os[:, :, :2], Of[:, :, :2])
    assert np.isnan(Os[:, :, 2:]).all()


# ---------------------------------------------------------------- planted mistakes

def _pins_pass(monkeypatch_ctx=None):
    """Run a compact set of the pins above; True iff all hold."""
    try:
        test_brute_force_tiny_config()
        test_matches_library_attention_causal_mtp()
        test_zero_query_gives_mean_of_values_and_log_n()
        test_single_token_cache_gives_that_value_row()
        test_constant_value_rows_give_that_row()
        test_empty_cache_gives_zero_and_minus_inf()
        test_sparse_matches_base2_prefill_equations()
        test_sparse_invalid_entries_are_removed()
    except AssertionError:
        return False
    return True


def test_pins_hold_for_the_real_oracle():
    assert _pins_pass()


def _mut_attend(kind):
    orig = odec.ref_attend_rows

    def bad(Q, K, dv, scale):
        if kind == "no_scale":
            return orig(Q, K, dv, 1.0)
        if kind == "value_last_cols":
            if K.shape[0] == 0:
                return orig(Q, K, dv, scale)
            o, l = orig(Q, K, dv, scale)
            S = scale * Q @ K.T
            E = np.exp(S - l[:, None])
            return E @ K[:, K.shape[1] - dv:], l
        if kind == "lse_base2":
            o, l = orig(Q, K, dv, scale)
            return o, l / math.log(2)
        if kind == "lse_no_max":
            o, l = orig(Q, K, dv, scale)
            if K.shape[0] == 0:
                return o, l
            return o, l - (scale * Q @ K.T).max(axis=1)
        if kind == "drop_last_key":
            return orig(Q, K[:-1], dv, scale)
        if kind == "rope_part_dropped":  # scores over the value columns only
            o, l = orig(Q[:, :dv], K[:, :dv], dv, scale)
            return o, l
        raise AssertionError(kind)
    return bad


@pytest.mark.parametrize("kind", ["no_scale", "value_last_cols", "lse_base2", "lse_no_max",
                                  "drop_last_key", "rope_part_dropped"])
def test_planted_mistake_in_attention_is_caught(monkeypatch, kind):
    monkeypatch.setattr(odec, "ref_attend_rows", _mut_attend(kind))
    assert not _pins_pass()


@pytest.mark.parametrize("kind", ["causal_off_by_one", "causal_top_left"])
def test_planted_mistake_in_causal_is_caught(monkeypatch, kind):
    orig = odec.visible_len

    def bad(L, s_q, i, causal):
        if not causal:
            return L
        if kind == "causal_off_by_one":
            return max(0, min(L, L - s_q + i))
        return max(0, min(L, i + 1))
    monkeypatch.setattr(odec, "visible_len", bad)
    assert not _pins_pass()


def test_planted_mistake_in_paging_is_caught(monkeypatch):
    orig = odec.ref_decode_paged

    def bad(q, kvcache, block_table, cache_seqlens, *a, **k):
        bt = block_table.clone() if isinstance(block_table, torch.Tensor) else block_table.copy()
        bt = bt.flip(-1) if isinstance(bt, torch.Tensor) else bt[:, ::-1]
        return orig(q, kvcache, bt, cache_seqlens, *a, **k)
    monkeypatch.setattr(oracle, "ref_decode_paged", bad)
    assert not _pins_pass()
