"""CPU-side checks of libmla.so: exports, the host scheduler, argument validation.

No GPU is needed: the scheduler is host code, and every decode call below is
rejected by argument validation before anything is enqueued (the pointers
passed are never dereferenced).
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import mla_paged_kv_amd as mla
from mla_paged_kv_amd import _binding as B
from oracle.schedule import ref_num_parts, ref_schedule, unpack_schedule as unpack

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.lib_path()):
        from mla_paged_kv_amd.build import build
        build()
    return B._load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for n in ["mla_get_metadata", "mla_get_metadata_device", "mla_sparse_prefill",
              "mla_decode_paged_fp8", "mla_decode_sparse_fp8", "mla_decode_paged", "mla_decode_sparse", "mla_workspace_bytes",
              "mla_strerror", "mla_last_error", "mla_version", "mla_default_num_parts",
              "mla_metadata_capacity"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", mla.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mla_\w+)$", out, flags=re.M))
    for n in header_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_version_and_strerror(lib):
    assert lib.mla_version() == 0x00010000
    assert lib.mla_strerror(0) == b"MLA_OK"
    assert lib.mla_strerror(-2) == b"MLA_E_NOTSUP"
    assert lib.mla_strerror(1) == b"MLA_W_ACTIVE_FALLBACK"


def _cpp_schedule(lens, P, rows):
    m = mla.mla_get_metadata(np.asarray(lens, dtype=np.int32), 1, rows, num_parts=P, num_cus=0,
                             upload=False)
    return m.meta_host


@settings(max_examples=300, deadline=None)
@given(lens=st.lists(st.integers(0, 20000), min_size=0, max_size=60), P=st.integers(1, 1100),
       rows=st.integers(1, 256))
def test_cpp_scheduler_bit_exact_vs_reference(lib, lens, P, rows):
    np.testing.assert_array_equal(_cpp_schedule(lens, P, rows), ref_schedule(lens, P, rows))


def test_cpp_scheduler_bit_exact_at_config_shapes(lib):
    from synth.configs import WORKLOADS, rng_for
    for k, spec in WORKLOADS.items():
        if spec["kind"] == "dense":
            lens = spec.get("seqlens")
            if lens is None:
                lens = spec["seqlen_sampler"](rng_for(1000 + k))
            rows = spec["s_q"] * spec["h_q"]
            units = lens
        else:
            rows = spec["active_h_q"]
            units = [spec["topk"]] * (spec["B"] * spec["s_q"])
        for cus in (256, 304, 80):
            P = ref_num_parts(rows, cus)
            assert lib.mla_default_num_parts(rows, cus) == P
            np.testing.assert_array_equal(_cpp_schedule(units, P, rows), ref_schedule(units, P, rows))


def test_sparse_mode_units_are_query_tokens(lib):
    m = mla.mla_get_metadata([5, 5, 5], 2, 64, topk=300, active_h_q=16, num_cus=256, upload=False)
    assert m.num_units == 6 and m.rows == 16
    np.testing.assert_array_equal(m.meta_host, ref_schedule([300] * 6, ref_num_parts(16, 256), 16))


def test_active_heads_fail_closed(lib):
    with pytest.warns(UserWarning):
        m = mla.mla_get_metadata(None or [10], 1, 64, topk=64, active_h_q=12, num_cus=256, upload=False)
    assert m.rows == 64
    m = mla.mla_get_metadata([10], 1, 64, topk=64, active_h_q=16, num_cus=256, upload=False)
    assert m.rows == 16
    m = mla.mla_get_metadata([10], 2, 32, active_h_q=8, num_cus=256, upload=False)
    assert m.rows == 16 and m.heads == 8
    with pytest.warns(UserWarning):
        m = mla.mla_get_metadata([10], 1, 64, topk=64, active_h_q=72, num_cus=256, upload=False)
    assert m.rows == 64


def _raw_meta(lib, lens, P=4, rows=16):
    cap = lib.mla_metadata_capacity(len(lens), P)
    meta = np.zeros(cap, dtype=np.int32)
    info = B.MlaSchedInfo()
    sl = np.asarray(lens, dtype=np.int32)
    rc = lib.mla_get_metadata(sl.ctypes.data, len(lens), 1, rows, 1, 0, 0, 0, P,
                              meta.ctypes.data, cap, ctypes.byref(info))
    return rc, meta, info


def test_get_metadata_errors(lib):
    info = B.MlaSchedInfo()
    meta = np.zeros(8, dtype=np.int32)
    sl = np.asarray([100, 200], dtype=np.int32)
    # capacity too small
    assert lib.mla_get_metadata(sl.ctypes.data, 2, 1, 16, 1, 0, 0, 0, 4, meta.ctypes.data, 8,
                                ctypes.byref(info)) == -3
    big = np.zeros(1000, dtype=np.int32)
    # negative length
    neg = np.asarray([100, -1], dtype=np.int32)
    assert lib.mla_get_metadata(neg.ctypes.data, 2, 1, 16, 1, 0, 0, 0, 4, big.ctypes.data, 1000,
                                ctypes.byref(info)) == -1
    assert b"cache_seqlens[1]" in lib.mla_last_error()
    # h_q not a multiple of h_kv
    assert lib.mla_get_metadata(sl.ctypes.data, 2, 1, 15, 2, 0, 0, 0, 4, big.ctypes.data, 1000,
                                ctypes.byref(info)) == -1
    # neither num_cus nor num_parts
    assert lib.mla_get_metadata(sl.ctypes.data, 2, 1, 16, 1, 0, 0, 0, 0, big.ctypes.data, 1000,
                                ctypes.byref(info)) == -1
    # dense mode without lengths
    assert lib.mla_get_metadata(None, 2, 1, 16, 1, 0, 0, 0, 4, big.ctypes.data, 1000,
                                ctypes.byref(info)) == -1


FAKE = 1 << 20  # 16-byte aligned, never dereferenced: every call below fails validation


def test_get_metadata_device_rejects_before_launch(lib):
    """Every rejected call returns before the scheduler kernel is enqueued."""
    info = B.MlaSchedInfo()

    def call(sl=FAKE, batch=2, s_q=1, h_q=16, h_kv=1, topk=0, act=0, cus=0, P=4, meta=FAKE,
             cap=10 ** 6):
        return lib.mla_get_metadata_device(sl, batch, s_q, h_q, h_kv, topk, act, cus, P, meta, cap,
                                           ctypes.byref(info), None)

    assert call(meta=None) == -1                       # no output array
    assert call(sl=None) == -1                         # dense mode without lengths
    assert call(h_q=15, h_kv=2) == -1                  # h_q % h_kv
    assert call(P=0, cus=0) == -1                      # neither parts nor CUs
    assert call(s_q=0) == -1
    assert call(batch=4097) == -2                      # more units than one workgroup holds
    assert b"4096" in lib.mla_last_error()
    assert call(batch=1025, s_q=4, topk=64, sl=None) == -2   # sparse units = batch * s_q
    assert call(P=1025) == -2
    assert call(cap=int(lib.mla_metadata_capacity(2, 4)) - 1) == -3
    assert call(topk=(1 << 24) + 1, sl=None) == -1


def test_device_metadata_host_header_is_a_bound(lib):
    """The host header of device-built metadata bounds every count the
    reference scheduler produces for any lengths (checked on random lengths)."""
    rng = np.random.default_rng(5)
    for U, P in ((1, 1), (7, 3), (64, 256), (300, 16), (16, 1024)):
        for _ in range(20):
            lens = rng.integers(0, 20000, U)
            lens[rng.random(U) < 0.3] = rng.integers(0, 100)
            r = unpack(ref_schedule(lens.tolist(), P, 64))
            bound_segments = U + P - 1
            bound_slots = min(U + P - 1, 2 * (P - 1))
            assert r["num_parts"] <= P
            assert r["num_segments"] <= bound_segments
            assert r["total_slots"] <= bound_slots
            assert r["num_split_units"] <= min(U, P - 1)
            assert r["max_splits"] <= P
            assert r["total_ints"] <= lib.mla_metadata_capacity(U, P)


def _paged(lib, info, **kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, batch=2, s_q=1, h_q=16, h_kv=1, d_qk=576, dv=512,
             nblk=8, page=64, bt_stride=4, causal=0, scale=0.04, meta=FAKE, ws=None, ws_bytes=0,
             out=FAKE, lse=FAKE)
    a.update(kw)
    return lib.mla_decode_paged(a["q"], a["kv"], a["bt"], a["sl"], a["batch"], a["s_q"], a["h_q"],
                                a["h_kv"], a["d_qk"], a["dv"], a["nblk"], a["page"], a["bt_stride"],
                                a["causal"], a["scale"], a["meta"], ctypes.byref(info), a["ws"],
                                a["ws_bytes"], a["out"], a["lse"], None)


def test_decode_paged_rejects_bad_arguments(lib):
    rc, meta, info = _raw_meta(lib, [64, 200], P=512, rows=16)
    assert rc == 0 and info.total_slots > 0
    assert _paged(lib, info, h_kv=2, h_q=16) == -2          # h_kv != 1 not built
    assert _paged(lib, info, page=32) == -2                 # page size
    assert _paged(lib, info, d_qk=192) == -2                # MHA-mode head dims not built
    assert _paged(lib, info, dv=128, d_qk=576) == -2
    assert _paged(lib, info, dv=600) == -1                  # dv > d_qk
    assert _paged(lib, info, q=FAKE + 2) == -1              # misaligned
    assert _paged(lib, info, ws=None, ws_bytes=0) == -1     # splits need a workspace
    assert _paged(lib, info, ws=FAKE, ws_bytes=16) == -3    # workspace too small
    ws = lib.mla_workspace_bytes(ctypes.byref(info), 512)
    assert _paged(lib, info, ws=FAKE, ws_bytes=ws, batch=3) == -1   # metadata for 2 units
    assert _paged(lib, info, ws=FAKE, ws_bytes=ws, s_q=3) == -1     # rows 16 not a multiple of 3
    assert _paged(lib, info, ws=FAKE, ws_bytes=ws, h_q=8) == -1     # 16 heads > h_q
    assert _paged(lib, info, ws=FAKE, ws_bytes=ws, causal=2) == -1
    assert _paged(lib, info, ws=FAKE, ws_bytes=ws, scale=float("nan")) == -1
    assert _paged(lib, info, ws=FAKE, ws_bytes=ws, bt=None) == -1
    assert _paged(lib, info, ws=FAKE, ws_bytes=ws, bt_stride=0) == -1
    bad = B.MlaSchedInfo.from_buffer_copy(info)
    bad.row_blocks = 7
    assert _paged(lib, bad, ws=FAKE, ws_bytes=ws) == -1     # malformed header
    assert b"row_blocks" in lib.mla_last_error()


def _paged_noalloc(lib, info, **kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, batch=2, s_q=1, h_q=16, h_kv=1, d_qk=576, dv=512,
             nblk=8, page=64, bt_stride=4, causal=0, scale=0.04, meta=FAKE, out=FAKE, lse=FAKE)
    a.update(kw)
    return lib.mla_decode_paged_noalloc(a["q"], a["kv"], a["bt"], a["sl"], a["batch"], a["s_q"],
                                        a["h_q"], a["h_kv"], a["d_qk"], a["dv"], a["nblk"],
                                        a["page"], a["bt_stride"], a["causal"], a["scale"],
                                        a["meta"], ctypes.byref(info), a["out"], a["lse"], None)


def test_decode_paged_noalloc_checks_before_touching_the_gpu(lib):
    """The allocation-free variant runs mla_decode_paged's checks, then its
    own size limit, before any HIP call (so all of this runs without a GPU)."""
    rc, meta, info = _raw_meta(lib, [64, 200], P=512, rows=16)
    assert rc == 0 and info.total_slots > 0
    assert _paged_noalloc(lib, info, h_kv=2) == -2
    assert _paged_noalloc(lib, info, page=32) == -2
    assert _paged_noalloc(lib, info, q=FAKE + 2) == -1
    assert _paged_noalloc(lib, info, batch=3) == -1
    assert _paged_noalloc(lib, info, causal=2) == -1
    assert _paged_noalloc(lib, info, bt=None) == -1
    assert _paged_noalloc(lib, info, batch=0) == 0           # nothing to do, nothing touched
    # a schedule whose split partials exceed the static array is refused
    rc, meta, info = _raw_meta(lib, [65536] * 4, P=1024, rows=128)
    assert rc == 0
    assert lib.mla_workspace_bytes(ctypes.byref(info), 512) > (128 << 20)
    assert _paged_noalloc(lib, info, batch=4, h_q=128, nblk=4096, bt_stride=1024) == -3
    assert b"static scratch" in lib.mla_last_error()


def test_decode_sparse_rejects_bad_arguments(lib):
    cap = lib.mla_metadata_capacity(2, 8)
    meta = np.zeros(cap, dtype=np.int32)
    info = B.MlaSchedInfo()
    assert lib.mla_get_metadata(None, 2, 1, 64, 1, 2048, 16, 0, 8, meta.ctypes.data, cap,
                                ctypes.byref(info)) == 0
    ws = lib.mla_workspace_bytes(ctypes.byref(info), 512)

    def call(**kw):
        a = dict(q=FAKE, kv=FAKE, ix=FAKE, batch=2, s_q=1, h_q=64, h_kv=1, d_qk=512, dv=512,
                 nblk=64, page=64, topk=2048, scale=0.04, meta=FAKE, ws=FAKE, ws_bytes=ws,
                 out=FAKE, lse=FAKE)
        a.update(kw)
        return lib.mla_decode_sparse(a["q"], a["kv"], a["ix"], a["batch"], a["s_q"], a["h_q"],
                                     a["h_kv"], a["d_qk"], a["dv"], a["nblk"], a["page"],
                                     a["topk"], a["scale"], a["meta"], ctypes.byref(info),
                                     a["ws"], a["ws_bytes"], a["out"], a["lse"], None)

    assert call(ix=None) == -1
    assert call(topk=0) == -1
    assert call(batch=1) == -1       # metadata for 2 query tokens
    assert call(h_q=8) == -1         # 16 active heads > h_q
    assert call(d_qk=576, dv=576) == -2
    assert call(ws_bytes=ws - 4) == -3
    assert call(nblk=1 << 26) == -1  # rows would overflow int32


def test_workspace_bytes(lib):
    rc, meta, info = _raw_meta(lib, [64, 200], P=512, rows=16)
    n = lib.mla_workspace_bytes(ctypes.byref(info), 512)
    slots, rows = info.total_slots, info.rows
    # partial outputs, then partial LSEs and partial row maxima, each 256-byte aligned
    assert n == -(-slots * rows * 512 * 4 // 256) * 256 + 2 * (-(-slots * rows * 4 // 256) * 256)
    rc, meta, info = _raw_meta(lib, [64, 64], P=2, rows=16)
    assert info.total_slots == 0 and lib.mla_workspace_bytes(ctypes.byref(info), 512) == 0


def _sparse_meta(lib, units, heads=16, topk=2048, P=8):
    cap = lib.mla_metadata_capacity(units, P)
    meta = np.zeros(cap, dtype=np.int32)
    info = B.MlaSchedInfo()
    assert lib.mla_get_metadata(None, units, 1, 64, 1, topk, heads, 0, P, meta.ctypes.data, cap,
                                ctypes.byref(info)) == 0
    return meta, info


@pytest.mark.parametrize("name", ["mla_sparse_prefill", "mla_sparse_prefill_f16"])
def test_sparse_prefill_rejects_bad_arguments(lib, name):
    meta, info = _sparse_meta(lib, 3)
    ws = lib.mla_workspace_bytes(ctypes.byref(info), 512)

    def call(**kw):
        a = dict(q=FAKE, kv=FAKE, ix=FAKE, s_q=3, s_kv=4096, h_q=64, h_kv=1, d_qk=576, dv=512,
                 topk=2048, scale=0.04, ws=FAKE, ws_bytes=ws, out=FAKE, ml=FAKE, lse=FAKE)
        a.update(kw)
        return getattr(lib, name)(a["q"], a["kv"], a["ix"], a["s_q"], a["s_kv"], a["h_q"],
                                  a["h_kv"], a["d_qk"], a["dv"], a["topk"], a["scale"], FAKE,
                                  ctypes.byref(info), a["ws"], a["ws_bytes"], a["out"], a["ml"],
                                  a["lse"], None)

    assert call(s_kv=0) == -1
    assert call(s_kv=-5) == -1
    assert call(s_kv=(1 << 31) - 1) == -1                   # rows would overflow int32
    assert call(ix=None) == -1
    assert call(topk=0) == -1
    assert call(scale=0.0) == -1
    assert call(scale=float("inf")) == -1
    assert call(ml=FAKE + 2) == -1                          # max_logits misaligned
    assert call(s_q=2) == -1                                # metadata built for 3 query tokens
    assert b"units" in lib.mla_last_error()
    assert call(h_q=8) == -1                                # 16 active heads > h_q
    assert call(h_kv=2) == -2
    assert call(d_qk=576, dv=576) == -2
    assert call(ws_bytes=ws - 4) == -3
    assert call(ws=FAKE + 64) == -1                         # workspace not 256-aligned
    assert call(q=None) == -1
    assert call(lse=FAKE + 1) == -1
    assert call(s_q=0) == 0                                 # empty: nothing to launch


@pytest.mark.parametrize("suffix", ["", "_f16", "_fp8"])
def test_decode_variants_share_the_checks(lib, suffix):
    rc, meta, info = _raw_meta(lib, [64, 200], P=512, rows=16)
    ws = lib.mla_workspace_bytes(ctypes.byref(info), 512)
    for stage in ("decode", "splitkv"):
        fn = getattr(lib, f"mla_{stage}_paged{suffix}")
        args = [FAKE, FAKE, FAKE, FAKE, 2, 1, 16, 1, 576, 512, 8, 64, 4, 0, 0.04, FAKE,
                ctypes.byref(info), FAKE, ws, FAKE, FAKE, None]
        bad = list(args)
        bad[11] = 32                                        # page size
        assert fn(*bad) == -2
        bad = list(args)
        bad[4] = 3                                          # metadata for 2 units
        assert fn(*bad) == -1
        bad = list(args)
        bad[18] = ws - 1
        assert fn(*bad) == -3
        bad = list(args)
        bad[8], bad[4] = 512, 0   # d_qk 512, empty batch: the FP8 format needs 576, else no-op
        assert fn(*bad) == (-2 if suffix == "_fp8" else 0)
    smeta, sinfo = _sparse_meta(lib, 2)
    sws = lib.mla_workspace_bytes(ctypes.byref(sinfo), 512)
    for stage in ("decode", "splitkv"):
        fn = getattr(lib, f"mla_{stage}_sparse{suffix}")
        args = [FAKE, FAKE, FAKE, 2, 1, 64, 1, 576, 512, 64, 64, 2048, 0.04, FAKE,
                ctypes.byref(sinfo), FAKE, sws, FAKE, FAKE, None]
        bad = list(args)
        bad[2] = None                                       # indices
        assert fn(*bad) == -1
        bad = list(args)
        bad[11] = 0                                         # topk
        assert fn(*bad) == -1
        bad = list(args)
        bad[7] = 512
        bad[3] = 0
        assert fn(*bad) == (-2 if suffix == "_fp8" else 0)


@pytest.mark.parametrize("name", ["mla_combine", "mla_combine_f16"])
def test_combine_rejects_bad_arguments(lib, name):
    fn = getattr(lib, name)
    rc, meta, info = _raw_meta(lib, [64, 200], P=512, rows=16)
    assert info.num_split_units > 0
    ws = lib.mla_workspace_bytes(ctypes.byref(info), 512)

    def call(pinfo=None, **kw):
        a = dict(meta=FAKE, batch=2, s_q=1, h_q=16, dv=512, sparse=0, ws=FAKE, ws_bytes=ws,
                 out=FAKE, lse=FAKE)
        a.update(kw)
        return fn(a["meta"], pinfo if pinfo is not None else ctypes.byref(info), a["batch"],
                  a["s_q"], a["h_q"], a["dv"], a["sparse"], a["ws"], a["ws_bytes"], a["out"],
                  a["lse"], None)

    assert fn(FAKE, None, 2, 1, 16, 512, 0, FAKE, ws, FAKE, FAKE, None) == -1   # null info
    assert call(dv=256) == -2
    assert call(sparse=2) == -1
    assert call(s_q=0) == -1
    assert call(batch=3) == -1                  # metadata for 2 units
    assert call(s_q=3) == -1                    # rows 16 not a multiple of 3
    assert call(h_q=8) == -1                    # 16 heads > h_q
    assert call(sparse=1, s_q=2) == -1          # sparse: 2 units != batch*s_q = 4
    assert call(ws=None) == -1
    assert call(ws=FAKE + 16) == -1             # not 256-aligned
    assert call(out=FAKE + 8) == -1
    assert call(ws_bytes=ws - 1) == -3
    assert call(batch=0) == -1                  # metadata for 2 units, batch 0
    bad = B.MlaSchedInfo.from_buffer_copy(info)
    bad.total_ints = 1
    assert call(pinfo=ctypes.byref(bad)) == -1
    # metadata without split units: nothing to combine, pointers never touched
    rc, meta1, info1 = _raw_meta(lib, [64, 64], P=2, rows=16)
    assert info1.num_split_units == 0
    assert fn(None, ctypes.byref(info1), 2, 1, 16, 512, 0, None, 0, None, None, None) == 0
