"""FP64 CPU oracle for paged MLA decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the ``mla_paged_kv_amd``
package, its C-ABI library or its HIP kernels) may import, call, link or run
anything in this folder; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do.  The oracle shares no code, header,
table or constant generator with the HIP path.

What it computes is the plain definition of softmax attention over a paged
latent cache, in float64, with a two-pass softmax (no online rescaling, no
splits):

* ``ref_decode_paged``   -- dense paged decode (FlashMLA usage page on
  deepep.org, "metadata + flash_mla_with_kvcache" example; upstream FlashMLA
  README embedded in the DeepLink-org/flashmla-optimization page, section
  "Usage / MLA Decoding").
* ``ref_decode_sparse``  -- token-level sparse decode through an ``indices``
  tensor (same README, "Sparse Attention (indices tensor)").
* ``fp8.dequant_rows``   -- the "FP8 with scale" cache row (upstream README,
  "FP8 KV Cache"): both decode functions accept such a cache and dequantize
  the rows they read.
* ``ref_sparse_prefill`` -- sparse MLA prefill (same README, "Sparse MLA
  Prefill": out, max_logits and a base-2 LSE, written from the softmax
  definition those outputs have).
* ``ref_schedule``       -- the reference tile scheduler.  The pages give only
  its purpose (metadata from sequence lengths and the head configuration that
  spreads variable-length work over compute units); the algorithm is this
  project's own written specification, implemented here from that text and,
  independently, in C++ in the library.  Its parity against the pages is
  therefore "parity unpinned": it is pinned only by the invariants that fully
  characterise the greedy partition (coverage, budget, maximality, slot
  numbering), checked in ``tests/test_oracle_schedule.py``.
"""
from . import fp8
from .decode import ref_decode_paged, ref_decode_sparse, ref_attend_rows
from .prefill import ref_sparse_prefill
from .schedule import (ref_schedule, ref_num_parts, unpack_schedule,
                       SPLIT_OVERHEAD_BLOCKS, PAGE_BLOCK)

__all__ = [
    "fp8",
    "ref_decode_paged",
    "ref_decode_sparse",
    "ref_attend_rows",
    "ref_sparse_prefill",
    "ref_schedule",
    "ref_num_parts",
    "unpack_schedule",
    "SPLIT_OVERHEAD_BLOCKS",
    "PAGE_BLOCK",
]
