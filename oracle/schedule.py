"""Reference split-KV tile scheduler (pure Python, integer only).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The pages say what the scheduler is for and when it runs -- metadata computed
from the cache sequence lengths and the head configuration, once, then reused by
every layer's decode call, so that variable-length work is spread over the
GPU's compute units (FlashMLA usage page on deepep.org, the ``get_mla_metadata``
example and the "metadata generation" and "Tile Scheduler" paragraphs; upstream
FlashMLA README embedded in the DeepLink-org/flashmla-optimization page,
"Usage / MLA Decoding", six-argument form with ``h_q`` and ``topk``).  They do
not give the algorithm.  The algorithm below is this project's written
specification; this file implements it from that text, and the C++ library
implements it again, independently.  They must agree bit for bit.

Specification
-------------
Work units: dense decode -> one unit per request b with length
``cache_seqlens[b]``; sparse decode -> one unit per query token (b, i),
``u = b * s_q + i``, with length ``topk``.  A unit of length ``len`` has
``nb = ceil(len / 64)`` blocks (64-token pages, or 64-index chunks).

Given a target part count ``P >= 1`` and a per-segment overhead ``F`` (in block
units; F = 5):

    total = sum(nb[u] + F)
    quota = ceil(total / P) + F

Parts are filled in order by a cursor (u, j) that starts at (0, 0).  Each part
starts with a budget ``rem = quota`` and repeats:

* if no unit is left, stop;
* ``need = nb[u] - j + F``; if ``need <= rem``, emit segment (u, j, nb[u]),
  ``rem -= need``, move to the next unit with j = 0;
* else if ``rem > F``, emit (u, j, j + rem - F), advance j by ``rem - F`` and
  close the part;
* else close the part.

Parts are opened until every unit is consumed; the walk provably uses at most P
parts.  A unit cut into k >= 2 segments is "split": its segments get
consecutive workspace slots, numbered over split units in unit order; an unsplit
unit's single segment gets slot -1 (written straight to the output).

Default part count: ``rows`` query rows per unit are processed ``G(rows)``
per workgroup, where G(rows) = 128 if rows > 64, else 64, and one workgroup is
resident per compute unit (a workgroup's tile buffers
fill most of the LDS), so that every part starts at once:
``row_blocks = ceil(rows / G(rows))`` and ``P = max(1, num_cus // row_blocks)``.
G is a parameter of the specification (``rows_per_group``), not a property the
pages fix.

Metadata layout (int32):

    header[16] = num_parts, num_segments, total_slots, num_split_units,
                 max_splits, num_units, quota, total, target_parts, F,
                 row_blocks, rows, off_segs, off_num_splits, off_split_list,
                 total_ints
    part_ptr[num_parts + 1]      at 16: segment range of each part
    segs[num_segments][4]        at off_segs: (u, blk0, blk1, slot)
    num_splits[num_units + 1]    at off_num_splits: cumulative segment counts
    split_list[num_split_units][2] at off_split_list: (u, first slot)
"""
from __future__ import annotations

import numpy as np

PAGE_BLOCK = 64
SPLIT_OVERHEAD_BLOCKS = 5
WORKGROUPS_PER_CU = 1
HEADER_INTS = 16


def rows_per_group(rows: int) -> int:
    """G(rows): query rows per workgroup (see the specification above)."""
    return 128 if rows > 64 else 64


def ref_row_blocks(rows: int, group=None) -> int:
    g = rows_per_group(rows) if group is None else group
    return -(-rows // g)


def ref_num_parts(rows: int, num_cus: int, group=None) -> int:
    return max(1, (WORKGROUPS_PER_CU * num_cus) // ref_row_blocks(rows, group))


def ref_schedule(lens, target_parts: int, rows: int, group=None) -> np.ndarray:
    """Build the metadata array for unit lengths ``lens`` and ``target_parts``
    parts; ``group`` overrides G(rows) (the header's row_blocks only)."""
    lens = [int(x) for x in lens]
    assert target_parts >= 1 and rows >= 1 and all(x >= 0 for x in lens)
    F = SPLIT_OVERHEAD_BLOCKS
    U = len(lens)
    nb = [-(-x // PAGE_BLOCK) for x in lens]
    total = sum(n + F for n in nb)
    quota = -(-total // target_parts) + F

    segs = []  # (u, blk0, blk1)
    part_ptr = [0]
    u, j = 0, 0
    while u < U:
        rem = quota
        while u < U:
            need = nb[u] - j + F
            if need <= rem:
                segs.append((u, j, nb[u]))
                rem -= need
                u, j = u + 1, 0
            elif rem > F:
                take = rem - F
                segs.append((u, j, j + take))
                j += take
                break
            else:
                break
        part_ptr.append(len(segs))
    num_parts = len(part_ptr) - 1
    assert num_parts <= target_parts

    count = [0] * U
    for (su, _, _) in segs:
        count[su] += 1
    num_splits = [0]
    for x in count:
        num_splits.append(num_splits[-1] + x)
    slot_base = [-1] * U
    split_list = []
    nslots = 0
    for uu in range(U):
        if count[uu] >= 2:
            slot_base[uu] = nslots
            split_list.append((uu, nslots))
            nslots += count[uu]
    seg_rows = []
    seen = [0] * U
    for (su, b0, b1) in segs:
        slot = slot_base[su] + seen[su] if count[su] >= 2 else -1
        seen[su] += 1
        seg_rows.append((su, b0, b1, slot))

    S = len(seg_rows)
    off_segs = HEADER_INTS + num_parts + 1
    off_ns = off_segs + 4 * S
    off_sl = off_ns + U + 1
    total_ints = off_sl + 2 * len(split_list)
    row_blocks = ref_row_blocks(rows, group)
    header = [num_parts, S, nslots, len(split_list), max(count) if U else 0, U,
              quota, total, target_parts, F, row_blocks, rows,
              off_segs, off_ns, off_sl, total_ints]
    out = header + part_ptr
    for r in seg_rows:
        out.extend(r)
    out.extend(num_splits)
    for r in split_list:
        out.extend(r)
    assert len(out) == total_ints
    return np.asarray(out, dtype=np.int32)


def unpack_schedule(meta) -> dict:
    """Split a metadata array into named fields (views, for tests and tools)."""
    m = np.asarray(meta, dtype=np.int64)
    h = m[:HEADER_INTS]
    num_parts, S, nslots, nsu, max_splits, U = (int(x) for x in h[:6])
    off_segs, off_ns, off_sl, total_ints = (int(x) for x in h[12:16])
    return dict(
        num_parts=num_parts, num_segments=S, total_slots=nslots, num_split_units=nsu,
        max_splits=max_splits, num_units=U, quota=int(h[6]), total=int(h[7]),
        target_parts=int(h[8]), F=int(h[9]), row_blocks=int(h[10]), rows=int(h[11]),
        part_ptr=m[HEADER_INTS:HEADER_INTS + num_parts + 1],
        segs=m[off_segs:off_segs + 4 * S].reshape(S, 4),
        num_splits=m[off_ns:off_ns + U + 1],
        split_list=m[off_sl:off_sl + 2 * nsu].reshape(nsu, 2),
        total_ints=total_ints,
    )
