"""ctypes marshalling for libmla.so (argument checks, allocation, pointers)."""
from __future__ import annotations

import ctypes
import math
import os
import warnings

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmla.so")

MLA_OK = 0
MLA_W_ACTIVE_FALLBACK = 1

_HEADER_FIELDS = [
    "num_parts", "num_segments", "total_slots", "num_split_units", "max_splits", "num_units",
    "quota", "total_cost", "target_parts", "overhead", "row_blocks", "rows", "off_segs",
    "off_num_splits", "off_split_list", "total_ints",
]


class MlaSchedInfo(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in _HEADER_FIELDS]


class MLAError(RuntimeError):
    """A negative return code from libmla.so."""

    def __init__(self, code: int, what: str, detail: str):
        super().__init__(f"{what}: {detail} (code {code})")
        self.code = code


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build the HIP library first "
            "(python -m mla_paged_kv_amd.build). There is no fallback path.")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, sz, vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    pinfo = ctypes.POINTER(MlaSchedInfo)
    lib.mla_version.restype = i32
    lib.mla_strerror.restype = ctypes.c_char_p
    lib.mla_strerror.argtypes = [ctypes.c_int]
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_default_num_parts.restype = i32
    lib.mla_default_num_parts.argtypes = [i32, i32]
    lib.mla_metadata_capacity.restype = sz
    lib.mla_metadata_capacity.argtypes = [i32, i32]
    lib.mla_get_metadata.restype = ctypes.c_int
    lib.mla_get_metadata.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, pinfo]
    lib.mla_get_metadata_device.restype = ctypes.c_int
    lib.mla_get_metadata_device.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz,
                                            pinfo, vp]
    lib.mla_workspace_bytes.restype = sz
    lib.mla_workspace_bytes.argtypes = [pinfo, i32]
    lib.mla_decode_paged.restype = ctypes.c_int
    lib.mla_decode_paged.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                     i32, ctypes.c_float, vp, pinfo, vp, sz, vp, vp, vp]
    lib.mla_decode_sparse.restype = ctypes.c_int
    lib.mla_decode_sparse.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                      ctypes.c_float, vp, pinfo, vp, sz, vp, vp, vp]
    lib.mla_splitkv_paged.restype = ctypes.c_int
    lib.mla_splitkv_paged.argtypes = lib.mla_decode_paged.argtypes
    lib.mla_splitkv_sparse.restype = ctypes.c_int
    lib.mla_splitkv_sparse.argtypes = lib.mla_decode_sparse.argtypes
    for name in ("mla_decode_paged_fp8", "mla_splitkv_paged_fp8"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = lib.mla_decode_paged.argtypes
    for name in ("mla_decode_sparse_fp8", "mla_splitkv_sparse_fp8"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = lib.mla_decode_sparse.argtypes
    for name in ("mla_decode_paged_f16", "mla_splitkv_paged_f16"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = lib.mla_decode_paged.argtypes
    for name in ("mla_decode_sparse_f16", "mla_splitkv_sparse_f16"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = lib.mla_decode_sparse.argtypes
    for name in ("mla_sparse_prefill", "mla_sparse_prefill_f16"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                       ctypes.c_float, vp, pinfo, vp, sz, vp, vp, vp, vp]
    lib.mla_decode_paged_noalloc.restype = ctypes.c_int
    lib.mla_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                             i32, i32, i32, ctypes.c_float, vp, pinfo, vp, vp, vp]
    lib.mla_combine.restype = ctypes.c_int
    lib.mla_combine.argtypes = [vp, pinfo, i32, i32, i32, i32, i32, vp, sz, vp, vp, vp]
    lib.mla_combine_f16.restype = ctypes.c_int
    lib.mla_combine_f16.argtypes = lib.mla_combine.argtypes
    _lib = lib
    return lib


def _check(rc: int, what: str) -> int:
    if rc < 0:
        lib = _load()
        raise MLAError(rc, what, f"{lib.mla_strerror(rc).decode()}: {lib.mla_last_error().decode()}")
    return rc


class Metadata:
    """Tile-scheduler output: host header + arrays, and the device copy.

    For metadata built on the device (:func:`mla_get_metadata_device`),
    ``meta_host`` is None and ``info`` holds upper bounds; :meth:`exact`
    copies the device array to the host (synchronising)."""

    def __init__(self, info: MlaSchedInfo, meta_host, meta_dev, *, sparse: bool,
                 batch: int, s_q: int, h_q: int, topk: int, device_built: bool = False):
        self.info = info
        self.meta_host = meta_host
        self.meta_dev = meta_dev
        self.sparse = sparse
        self.device_built = device_built
        self.batch, self.s_q, self.h_q, self.topk = batch, s_q, h_q, topk

    def __getattr__(self, name):
        if name in _HEADER_FIELDS:
            return getattr(self.info, name)
        raise AttributeError(name)

    @property
    def heads(self) -> int:
        return self.info.rows if self.sparse else self.info.rows // self.s_q

    def exact(self) -> np.ndarray:
        """The metadata array as the decode kernels see it (header + arrays)."""
        if not self.device_built:
            return self.meta_host
        m = self.meta_dev.cpu().numpy()
        return m[:max(16, int(m[15]))]

    @property
    def num_splits(self) -> np.ndarray:
        """Cumulative segment count per unit, [num_units + 1]."""
        m = self.exact()
        o = int(m[13])
        return m[o:o + self.info.num_units + 1]

    @property
    def segments(self) -> np.ndarray:
        m = self.exact()
        o = int(m[12])
        return m[o:o + 4 * int(m[1])].reshape(-1, 4)

    def blocks_needed(self) -> int:
        """Most block-table columns any segment reaches (host-built metadata;
        computed once)."""
        if getattr(self, "_blocks_needed", None) is None:
            segs = self.segments
            self._blocks_needed = int(segs[:, 2].max()) if len(segs) else 0
        return self._blocks_needed

    def workspace_bytes(self, dv: int = 512) -> int:
        return int(_load().mla_workspace_bytes(ctypes.byref(self.info), dv))


def _num_cus(device) -> int:
    return int(torch.cuda.get_device_properties(device).multi_processor_count)


def mla_get_metadata(cache_seqlens, s_q: int, h_q: int, h_kv: int = 1, topk: int = 0,
                     active_h_q: int = 0, num_parts: int = 0, num_cus: int | None = None,
                     device=None, upload: bool = True) -> Metadata:
    """Tile scheduler.  ``cache_seqlens``: [batch] ints (host or device; a device
    tensor is copied to the host, which synchronises).  ``topk > 0`` selects
    sparse mode.  Returns a :class:`Metadata` whose ``meta_dev`` lives on
    ``device`` (default: the current CUDA device) unless ``upload`` is False."""
    lib = _load()
    if isinstance(cache_seqlens, torch.Tensor):
        if device is None and cache_seqlens.is_cuda:
            device = cache_seqlens.device
        sl = cache_seqlens.detach().to("cpu", torch.int32).contiguous().numpy()
    else:
        sl = np.ascontiguousarray(np.asarray(cache_seqlens, dtype=np.int32))
    batch = int(sl.shape[0])
    if upload and device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    if num_cus is None:
        num_cus = _num_cus(device) if (num_parts == 0) else 0
    units = batch * s_q if topk > 0 else batch
    if num_parts > 0:
        target = num_parts
    else:
        # size for the requested head count and for the all-heads fallback
        per_unit = s_q if topk == 0 else 1
        target = max(int(lib.mla_default_num_parts(per_unit * h, max(1, num_cus)))
                     for h in {max(1, active_h_q or h_q), h_q})
    cap = int(lib.mla_metadata_capacity(units, max(1, target)))
    meta = np.zeros(cap, dtype=np.int32)
    info = MlaSchedInfo()
    rc = lib.mla_get_metadata(sl.ctypes.data if batch else None, batch, s_q, h_q, h_kv, topk,
                              active_h_q, int(num_cus), num_parts, meta.ctypes.data, cap,
                              ctypes.byref(info))
    _check(rc, "mla_get_metadata")
    if rc == MLA_W_ACTIVE_FALLBACK:
        warnings.warn(f"active_h_q={active_h_q} invalid for h_q={h_q}: all heads are computed")
    meta = meta[:info.total_ints].copy()
    meta_dev = torch.from_numpy(meta).to(device) if upload else None
    return Metadata(info, meta, meta_dev, sparse=topk > 0, batch=batch, s_q=s_q, h_q=h_q, topk=topk)


def mla_get_metadata_device(cache_seqlens, s_q: int, h_q: int, h_kv: int = 1, topk: int = 0,
                            active_h_q: int = 0, num_parts: int = 0, num_cus: int | None = None,
                            batch: int | None = None, device=None, meta_out=None) -> Metadata:
    """Tile scheduler on the GPU, enqueued on the current stream (no
    synchronisation; capturable in a CUDA/HIP graph).  ``cache_seqlens``: [batch]
    int32 device tensor (may be None in sparse mode, then give ``batch``).
    ``meta_out``: optional preallocated int32 device tensor of at least
    ``mla_metadata_capacity`` ints (reused across graph replays)."""
    lib = _load()
    if cache_seqlens is not None:
        _need(isinstance(cache_seqlens, torch.Tensor) and cache_seqlens.is_cuda
              and cache_seqlens.dtype == torch.int32 and cache_seqlens.is_contiguous()
              and cache_seqlens.dim() == 1, "cache_seqlens must be a contiguous int32 [B] GPU tensor")
        batch = int(cache_seqlens.shape[0])
        device = cache_seqlens.device
    _need(batch is not None, "give cache_seqlens or batch")
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    if num_cus is None:
        num_cus = _num_cus(device) if num_parts == 0 else 0
    units = batch * s_q if topk > 0 else batch
    if num_parts > 0:
        target = num_parts
    else:
        per_unit = s_q if topk == 0 else 1
        target = max(int(lib.mla_default_num_parts(per_unit * h, max(1, num_cus)))
                     for h in {max(1, active_h_q or h_q), h_q})
    cap = int(lib.mla_metadata_capacity(units, max(1, target)))
    if meta_out is None:
        meta_out = torch.empty(cap, dtype=torch.int32, device=device)
    _need(meta_out.dtype == torch.int32 and meta_out.is_cuda and meta_out.is_contiguous(),
          "meta_out must be a contiguous int32 GPU tensor")
    info = MlaSchedInfo()
    rc = lib.mla_get_metadata_device(_ptr(cache_seqlens), batch, s_q, h_q, h_kv, topk, active_h_q,
                                     int(num_cus), num_parts, _ptr(meta_out), meta_out.numel(),
                                     ctypes.byref(info), _stream(device))
    _check(rc, "mla_get_metadata_device")
    if rc == MLA_W_ACTIVE_FALLBACK:
        warnings.warn(f"active_h_q={active_h_q} invalid for h_q={h_q}: all heads are computed")
    return Metadata(info, None, meta_out, sparse=topk > 0, batch=batch, s_q=s_q, h_q=h_q,
                    topk=topk, device_built=True)


def mla_workspace_bytes(meta: Metadata, dv: int = 512) -> int:
    return meta.workspace_bytes(dv)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _prep_outputs(q, meta, dv, workspace, out, lse):
    B, s_q, h_q, _ = q.shape
    if out is None:
        out = torch.empty((B, s_q, h_q, dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=q.device)
    _need(out.shape == (B, s_q, h_q, dv) and out.dtype == q.dtype and out.is_contiguous(),
          "out must be contiguous [B, s_q, h_q, dv] of q's dtype")
    _need(lse.shape == (B, s_q, h_q) and lse.dtype == torch.float32 and lse.is_contiguous(),
          "lse must be contiguous fp32 [B, s_q, h_q]")
    need = meta.workspace_bytes(dv)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return out, lse, workspace, ws_bytes


FP8_ROW_BYTES = 656  # "FP8 with scale" cache row: 512 e4m3, 4 fp32 scales, 64 bf16


_ELEM = {torch.bfloat16: "bf16", torch.float16: "f16"}


def _kv_format(q, kvcache):
    """'bf16', 'f16' (q, cache and out fp16) or 'fp8' (bf16 q, uint8 cache rows
    of 656 bytes, d_qk must be 576)."""
    if kvcache.dtype == torch.uint8:
        _need(q.dtype == torch.bfloat16, "an FP8 cache takes a bf16 q")
        _need(kvcache.shape[-1] == FP8_ROW_BYTES, "an FP8 cache has 656-byte rows")
        _need(q.shape[-1] == 576, "the FP8 cache format needs d_qk = 576")
        return "fp8"
    _need(q.dtype in _ELEM and kvcache.dtype == q.dtype,
          "q and kvcache must both be bf16 or both fp16 (or kvcache uint8 FP8-with-scale rows)")
    _need(kvcache.shape[-1] == q.shape[-1], "kvcache row width must equal q's d_qk")
    return _ELEM[q.dtype]


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def mla_decode_paged(q, kvcache, block_table, cache_seqlens, dv: int, meta: Metadata,
                     causal: bool = False, softmax_scale: float | None = None,
                     workspace=None, out=None, lse=None, stage: str = "all"):
    """Dense paged decode; returns (out [B, s_q, h_q, dv] bf16, lse [B, s_q, h_q] fp32).

    ``stage="split"`` runs only the split-KV kernel (then call
    :func:`mla_combine` with the same workspace, out and lse)."""
    lib = _load()
    _need(q.dim() == 4 and kvcache.dim() == 4, "q is [B, s_q, h_q, d_qk], kvcache [blocks, 64, h_kv, d_qk]")
    fmt = _kv_format(q, kvcache)
    sfx = {"bf16": "", "f16": "_f16", "fp8": "_fp8"}[fmt]
    fn = getattr(lib, ("mla_decode_paged" if stage == "all" else "mla_splitkv_paged") + sfx)
    _need(q.is_cuda and kvcache.is_cuda and block_table.is_cuda and cache_seqlens.is_cuda,
          "all tensors must be on the GPU")
    _need(q.is_contiguous() and kvcache.is_contiguous() and block_table.is_contiguous()
          and cache_seqlens.is_contiguous(), "tensors must be contiguous")
    _need(block_table.dtype == torch.int32 and cache_seqlens.dtype == torch.int32,
          "block_table and cache_seqlens must be int32")
    _need(not meta.sparse, "metadata was built for sparse decode")
    B, s_q, h_q, d_qk = q.shape
    nblk, page, h_kv, _ = kvcache.shape
    _need(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be [B, max_blocks]")
    _need(cache_seqlens.shape == (B,), "cache_seqlens must be [B]")
    if not meta.device_built:  # (device metadata is not read back: no synchronisation)
        _need(meta.blocks_needed() <= block_table.shape[1],
              "cache_seqlens of the metadata need more blocks than block_table has columns")
    if softmax_scale is None:
        softmax_scale = d_qk ** -0.5
    out, lse, workspace, ws_bytes = _prep_outputs(q, meta, dv, workspace, out, lse)
    rc = fn(_ptr(q), _ptr(kvcache), _ptr(block_table), _ptr(cache_seqlens), B,
                              s_q, h_q, h_kv, d_qk, dv, nblk, page, block_table.shape[1],
                              1 if causal else 0, float(softmax_scale), _ptr(meta.meta_dev),
                              ctypes.byref(meta.info), _ptr(workspace), ws_bytes, _ptr(out),
                              _ptr(lse), _stream(q.device))
    _check(rc, "mla_decode_paged")
    if stage == "split":
        return out, lse, workspace
    return out, lse


def mla_decode_paged_noalloc(q, kvcache, block_table, cache_seqlens, dv: int, meta: Metadata,
                             causal: bool = False, softmax_scale: float | None = None,
                             out=None, lse=None):
    """Dense paged decode (bf16) whose split partials live in the library's
    static device array: the C call allocates nothing.  Pass ``out`` and
    ``lse`` to allocate nothing here either.  Returns (out, lse)."""
    lib = _load()
    _need(q.dim() == 4 and kvcache.dim() == 4, "q is [B, s_q, h_q, d_qk], kvcache [blocks, 64, h_kv, d_qk]")
    _need(q.dtype == torch.bfloat16 and kvcache.dtype == torch.bfloat16, "q and kvcache must be bf16")
    _need(q.is_cuda and kvcache.is_cuda and block_table.is_cuda and cache_seqlens.is_cuda,
          "all tensors must be on the GPU")
    _need(q.is_contiguous() and kvcache.is_contiguous() and block_table.is_contiguous()
          and cache_seqlens.is_contiguous(), "tensors must be contiguous")
    _need(block_table.dtype == torch.int32 and cache_seqlens.dtype == torch.int32,
          "block_table and cache_seqlens must be int32")
    _need(not meta.sparse, "metadata was built for sparse decode")
    B, s_q, h_q, d_qk = q.shape
    nblk, page, h_kv, _ = kvcache.shape
    _need(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be [B, max_blocks]")
    _need(cache_seqlens.shape == (B,), "cache_seqlens must be [B]")
    if not meta.device_built:
        _need(meta.blocks_needed() <= block_table.shape[1],
              "cache_seqlens of the metadata need more blocks than block_table has columns")
    if softmax_scale is None:
        softmax_scale = d_qk ** -0.5
    if out is None:
        out = torch.empty((B, s_q, h_q, dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=q.device)
    _need(out.shape == (B, s_q, h_q, dv) and out.dtype == q.dtype and out.is_contiguous(),
          "out must be contiguous [B, s_q, h_q, dv] bf16")
    _need(lse.shape == (B, s_q, h_q) and lse.dtype == torch.float32 and lse.is_contiguous(),
          "lse must be contiguous fp32 [B, s_q, h_q]")
    rc = lib.mla_decode_paged_noalloc(
        _ptr(q), _ptr(kvcache), _ptr(block_table), _ptr(cache_seqlens), B, s_q, h_q, h_kv, d_qk,
        dv, nblk, page, block_table.shape[1], 1 if causal else 0, float(softmax_scale),
        _ptr(meta.meta_dev), ctypes.byref(meta.info), _ptr(out), _ptr(lse), _stream(q.device))
    _check(rc, "mla_decode_paged_noalloc")
    return out, lse


def mla_decode_sparse(q, kvcache, indices, dv: int, meta: Metadata,
                      softmax_scale: float | None = None, workspace=None, out=None, lse=None,
                      stage: str = "all"):
    """Top-k sparse decode; heads past the metadata's active count are not written."""
    lib = _load()
    _need(q.dim() == 4 and kvcache.dim() == 4 and indices.dim() == 3, "bad ranks")
    fmt = _kv_format(q, kvcache)
    sfx = {"bf16": "", "f16": "_f16", "fp8": "_fp8"}[fmt]
    fn = getattr(lib, ("mla_decode_sparse" if stage == "all" else "mla_splitkv_sparse") + sfx)
    _need(indices.dtype == torch.int32, "indices must be int32")
    _need(q.is_cuda and kvcache.is_cuda and indices.is_cuda, "all tensors must be on the GPU")
    _need(q.is_contiguous() and kvcache.is_contiguous() and indices.is_contiguous(),
          "tensors must be contiguous")
    _need(meta.sparse, "metadata was built for dense decode")
    B, s_q, h_q, d_qk = q.shape
    nblk, page, h_kv, _ = kvcache.shape
    _need(indices.shape[:2] == (B, s_q), "indices must be [B, s_q, topk]")
    topk = indices.shape[2]
    _need(topk == meta.topk, f"indices topk {topk} != metadata topk {meta.topk}")
    if softmax_scale is None:
        softmax_scale = d_qk ** -0.5
    out, lse, workspace, ws_bytes = _prep_outputs(q, meta, dv, workspace, out, lse)
    rc = fn(_ptr(q), _ptr(kvcache), _ptr(indices), B, s_q, h_q, h_kv, d_qk, dv,
                               nblk, page, topk, float(softmax_scale), _ptr(meta.meta_dev),
                               ctypes.byref(meta.info), _ptr(workspace), ws_bytes, _ptr(out),
                               _ptr(lse), _stream(q.device))
    _check(rc, "mla_decode_sparse")
    if stage == "split":
        return out, lse, workspace
    return out, lse


def mla_combine(meta: Metadata, out, lse, workspace, dv: int = 512):
    """LSE-merge the split partials in ``workspace`` into ``out``/``lse``."""
    lib = _load()
    B, s_q, h_q, _ = out.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _need(out.dtype in _ELEM, "out must be bf16 or fp16")
    fn = lib.mla_combine_f16 if out.dtype == torch.float16 else lib.mla_combine
    rc = fn(_ptr(meta.meta_dev), ctypes.byref(meta.info), B, s_q, h_q, dv,
                         1 if meta.sparse else 0, _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                         _stream(out.device))
    _check(rc, "mla_combine")
    return out, lse


def mla_sparse_prefill(q, kv, indices, sm_scale: float, dv: int = 512, meta: Metadata | None = None,
                       num_parts: int = 0, workspace=None, out=None, max_logits=None, lse=None):
    """Sparse MLA prefill: q [s_q, h_q, d_qk], kv [s_kv, 1, d_qk], indices
    [s_q, 1, topk] -> (out [s_q, h_q, dv] bf16, max_logits [s_q, h_q] fp32,
    lse [s_q, h_q] fp32 base 2).  ``meta``: sparse-mode metadata with batch =
    s_q and one query token each (built here when not given)."""
    lib = _load()
    _need(q.dim() == 3 and kv.dim() == 3 and indices.dim() == 3, "q [s_q,h_q,d], kv [s_kv,1,d], "
          "indices [s_q,1,topk]")
    _need(q.dtype in _ELEM and kv.dtype == q.dtype, "q and kv must both be bf16 or both fp16")
    _need(indices.dtype == torch.int32, "indices must be int32")
    _need(q.is_cuda and kv.is_cuda and indices.is_cuda, "all tensors must be on the GPU")
    _need(q.is_contiguous() and kv.is_contiguous() and indices.is_contiguous(),
          "tensors must be contiguous")
    s_q, h_q, d_qk = q.shape
    s_kv, h_kv, d_kv = kv.shape
    _need(d_kv == d_qk, "kv row width must equal q's d_qk")
    _need(indices.shape[:2] == (s_q, h_kv), "indices must be [s_q, h_kv, topk]")
    topk = indices.shape[2]
    if meta is None:
        meta = mla_get_metadata(np.zeros(s_q, np.int32), 1, h_q, h_kv, topk=topk,
                                num_parts=num_parts, device=q.device)
    _need(meta.sparse and meta.topk == topk, "metadata must be sparse-mode with the same topk")
    if out is None:
        out = torch.empty((s_q, h_q, dv), dtype=q.dtype, device=q.device)
    if max_logits is None:
        max_logits = torch.empty((s_q, h_q), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((s_q, h_q), dtype=torch.float32, device=q.device)
    need = meta.workspace_bytes(dv)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = lib.mla_sparse_prefill_f16 if q.dtype == torch.float16 else lib.mla_sparse_prefill
    rc = fn(_ptr(q), _ptr(kv), _ptr(indices), s_q, s_kv, h_q, h_kv, d_qk, dv,
                                topk, float(sm_scale), _ptr(meta.meta_dev), ctypes.byref(meta.info),
                                _ptr(workspace), ws_bytes, _ptr(out), _ptr(max_logits), _ptr(lse),
                                _stream(q.device))
    _check(rc, "mla_sparse_prefill")
    return out, max_logits, lse


# ---- the pages' call shape ------------------------------------------------

def get_mla_metadata(cache_seqlens, num_q_tokens_per_head_k: int, num_heads_k: int,
                     num_heads_q: int | None = None, is_fp8_kvcache: bool = False,
                     topk: int | None = None, active_h_q: int = 0):
    """The pages' ``get_mla_metadata(cache_seqlens, s_q*h_q//h_kv, h_kv[, h_q, is_fp8, topk])``.

    Returns ``(tile_scheduler_metadata, num_splits)``: the :class:`Metadata`
    object (pass it back as ``tile_scheduler_metadata``) and the cumulative
    per-unit segment counts on the device."""
    # (the schedule does not depend on the cache format)
    rows = int(num_q_tokens_per_head_k)
    if topk:
        _need(num_heads_q is not None, "sparse metadata needs num_heads_q")
        s_q = rows * num_heads_k // num_heads_q
        meta = mla_get_metadata(cache_seqlens, s_q, num_heads_q, num_heads_k, topk=int(topk),
                                active_h_q=active_h_q)
    else:
        h_q = num_heads_q if num_heads_q is not None else rows * num_heads_k
        s_q = rows * num_heads_k // h_q
        meta = mla_get_metadata(cache_seqlens, s_q, h_q, num_heads_k, active_h_q=active_h_q)
    ns = torch.from_numpy(meta.num_splits.copy()).to(meta.meta_dev.device)
    return meta, ns


def flash_mla_with_kvcache(q, k_cache, block_table, cache_seqlens, head_dim_v: int,
                           tile_scheduler_metadata: Metadata, num_splits=None,
                           softmax_scale: float | None = None, causal: bool = False,
                           is_fp8_kvcache: bool = False, indices=None):
    """The pages' ``flash_mla_with_kvcache``; returns (out, lse)."""
    if is_fp8_kvcache:
        if k_cache.dtype != torch.uint8:  # e.g. a float8 view of the same bytes
            k_cache = k_cache.view(torch.uint8)
        _need(k_cache.shape[-1] == FP8_ROW_BYTES, "is_fp8_kvcache: rows must be 656 bytes")
    else:
        _need(k_cache.dtype in _ELEM, "the cache must be bf16 or fp16 unless is_fp8_kvcache")
    if indices is not None:
        return mla_decode_sparse(q, k_cache, indices, head_dim_v, tile_scheduler_metadata,
                                 softmax_scale=softmax_scale)
    return mla_decode_paged(q, k_cache, block_table, cache_seqlens, head_dim_v,
                            tile_scheduler_metadata, causal=causal, softmax_scale=softmax_scale)


def flash_mla_sparse_fwd(q, kv, indices, sm_scale: float, d_v: int = 512):
    """The pages' ``flash_mla_sparse_fwd(q, kv, indices, sm_scale)``; returns
    (out, max_logits, lse) with a base-2 lse."""
    return mla_sparse_prefill(q, kv, indices, sm_scale, dv=d_v)
