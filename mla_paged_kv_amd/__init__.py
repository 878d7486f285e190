"""Paged MLA decode for MI355X (gfx950): Python binding of libmla.so.

Thin ctypes layer over the C ABI declared in ``include/mla.h``: it checks
tensor shapes and dtypes, allocates outputs and the split workspace with torch
(device memory and streams are all torch is used for) and passes raw pointers
and the current HIP stream.  Every step of the decode runs in the library's
HIP kernels; there is no fallback.  ``libmla.so`` is built in-tree by
``python -m mla_paged_kv_amd.build``; importing the package without it raises.

Entry points mirror the C ABI names:

* ``mla_get_metadata``   -- tile scheduler (host), once per decode step
* ``mla_get_metadata_device`` -- the same scheduler as a GPU kernel (no sync)
* ``mla_decode_paged``   -- dense paged decode, once per layer
* ``mla_decode_paged_noalloc`` -- the same without a workspace (static scratch)
* ``mla_decode_sparse``  -- top-k sparse decode, once per layer
* ``mla_sparse_prefill`` -- top-k sparse prefill (out, max_logits, base-2 lse)

and, for callers of the pages' Python API, ``get_mla_metadata`` /
``flash_mla_with_kvcache`` / ``flash_mla_sparse_fwd`` wrappers with the
pages' argument order.
"""
from ._binding import (  # noqa: F401
    MLAError,
    Metadata,
    flash_mla_sparse_fwd,
    flash_mla_with_kvcache,
    get_mla_metadata,
    lib_path,
    mla_combine,
    mla_decode_paged,
    mla_decode_paged_noalloc,
    mla_decode_sparse,
    mla_get_metadata,
    mla_get_metadata_device,
    mla_sparse_prefill,
    mla_workspace_bytes,
)

__all__ = [
    "MLAError",
    "Metadata",
    "flash_mla_sparse_fwd",
    "flash_mla_with_kvcache",
    "get_mla_metadata",
    "lib_path",
    "mla_combine",
    "mla_decode_paged",
    "mla_decode_paged_noalloc",
    "mla_decode_sparse",
    "mla_get_metadata",
    "mla_get_metadata_device",
    "mla_sparse_prefill",
    "mla_workspace_bytes",
]
