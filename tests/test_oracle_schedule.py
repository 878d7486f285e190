"""Pins for the reference tile scheduler (oracle/schedule.py).

The pages state the scheduler's purpose but not its algorithm, so there are no
printed values to pin against.  The written specification (greedy fill of
parts with budget ``quota``, split only when more than the per-segment
overhead is left) is pinned here by hand-worked small cases and by invariants
that together determine the greedy output uniquely: exact in-order coverage of
every unit, the per-part budget, maximality of every closed part, the part-count
bound, and the slot numbering.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle.schedule import (SPLIT_OVERHEAD_BLOCKS as F, ref_num_parts, ref_schedule,
                             unpack_schedule)


def test_hand_worked_tiny_workload():
    # lens 64, 200 -> blocks 1, 4; total = 6 + 9 = 15; 512 parts -> quota = 1 + 5 = 6.
    # part 0 takes unit 0 whole (need 6); unit 1 (need 9) is cut 1 block at a
    # time while need > 6, then its last block fits (need 6).
    m = ref_schedule([64, 200], 512, 16)
    assert m.tolist() == [
        5, 5, 4, 1, 4, 2, 6, 15, 512, 5, 1, 16, 22, 42, 45, 47,   # header
        0, 1, 2, 3, 4, 5,                                         # part_ptr
        0, 0, 1, -1, 1, 0, 1, 0, 1, 1, 2, 1, 1, 2, 3, 2, 1, 3, 4, 3,  # segs
        0, 1, 5,                                                  # num_splits
        1, 0,                                                     # split_list
    ]


def test_hand_worked_no_split_and_empty_unit():
    # lens 0, 130, 64 -> blocks 0, 3, 1; total = 5 + 8 + 6 = 19; P = 2 -> quota 15.
    # part 0: unit 0 (need 5, empty segment), unit 1 (need 8), then 2 left <= F: close.
    # part 1: unit 2.  128 rows per unit -> one 128-row workgroup per part.
    m = ref_schedule([0, 130, 64], 2, 128)
    assert m.tolist() == [
        2, 3, 0, 0, 1, 3, 15, 19, 2, 5, 1, 128, 19, 31, 35, 35,
        0, 2, 3,
        0, 0, 0, -1, 1, 0, 3, -1, 2, 0, 1, -1,
        0, 1, 2, 3,
    ]


def test_hand_worked_long_unit_even_cut():
    # 100 blocks, P = 4: total 105, quota 27 + 5 = 32 -> cuts of 27, 27, 27, then 19 fits.
    u = unpack_schedule(ref_schedule([6400], 4, 64))
    assert u["segs"].tolist() == [[0, 0, 27, 0], [0, 27, 54, 1], [0, 54, 81, 2], [0, 81, 100, 3]]
    assert u["num_parts"] == 4 and u["total_slots"] == 4 and u["max_splits"] == 4


def test_default_part_count():
    # G(rows) = 128 rows per workgroup above 64 rows, else 64
    assert ref_num_parts(16, 256) == 256
    assert ref_num_parts(33, 256) == 256
    assert ref_num_parts(64, 256) == 256
    assert ref_num_parts(65, 256) == 256
    assert ref_num_parts(128, 256) == 256
    assert ref_num_parts(129, 256) == 128
    assert ref_num_parts(256, 256) == 128
    assert ref_num_parts(257, 256) == 85
    assert ref_num_parts(10_000, 4) == 1
    # an explicit group size overrides the rule
    assert ref_num_parts(128, 256, group=64) == 128


def check_invariants(lens, P, rows, meta):
    u = unpack_schedule(meta)
    nb = [-(-x // 64) for x in lens]
    U = len(lens)
    total = sum(n + F for n in nb)
    quota = -(-total // P) + F
    assert u["num_units"] == U and u["quota"] == quota and u["total"] == total
    assert u["target_parts"] == P and u["F"] == F and u["rows"] == rows
    group = 128 if rows > 64 else 64
    assert u["row_blocks"] == -(-rows // group)
    segs = u["segs"]
    pp = u["part_ptr"]
    assert 0 <= u["num_parts"] <= P
    assert pp[0] == 0 and pp[-1] == len(segs) and np.all(np.diff(pp) >= 1)
    # coverage: units in order, each covered contiguously, exactly once
    cur_u, cur_j = 0, 0
    for (su, b0, b1, _) in segs.tolist():
        if su != cur_u:
            assert cur_j == nb[cur_u] and su == cur_u + 1
            cur_u, cur_j = su, 0
            # a unit only "finishes" when its last block is covered; empty units
            # have exactly one empty segment
        assert b0 == cur_j and b1 >= b0 and (b1 > b0 or nb[su] == 0)
        cur_j = b1
    if U:
        assert cur_u == U - 1 and cur_j == nb[-1]
        for uu in range(U):
            assert any(s[0] == uu for s in segs.tolist())
    else:
        assert len(segs) == 0
    # budget and maximality
    for p in range(u["num_parts"]):
        part = segs[pp[p]:pp[p + 1]].tolist()
        cost = sum(b1 - b0 + F for (_, b0, b1, _) in part)
        assert cost <= quota
        # only the last segment of a part may be a cut that leaves blocks behind
        for (su, b0, b1, _) in part[:-1]:
            assert b1 == nb[su]
        if p + 1 < u["num_parts"]:
            last = part[-1]
            nxt = segs[pp[p + 1]].tolist()
            if last[2] < nb[last[0]]:  # cut: the budget was used up exactly
                assert cost == quota and nxt[0] == last[0] and nxt[1] == last[2]
            else:  # closed at a unit end: the next unit did not fit, nor was a cut allowed
                left = quota - cost
                need = nb[nxt[0]] + F
                assert need > left and left <= F
    # slots and split bookkeeping
    counts = np.bincount(segs[:, 0], minlength=U) if U else np.zeros(0, dtype=int)
    assert u["num_splits"].tolist() == [0] + np.cumsum(counts).tolist()
    expected_slot = 0
    split_list = []
    for uu in range(U):
        mine = segs[segs[:, 0] == uu]
        if counts[uu] >= 2:
            split_list.append([uu, expected_slot])
            assert mine[:, 3].tolist() == list(range(expected_slot, expected_slot + counts[uu]))
            expected_slot += counts[uu]
        else:
            assert mine[:, 3].tolist() == [-1]
    assert u["total_slots"] == expected_slot
    assert u["split_list"].tolist() == split_list
    assert u["max_splits"] == (int(counts.max()) if U else 0)


@settings(max_examples=300, deadline=None)
@given(lens=st.lists(st.integers(0, 9000), min_size=0, max_size=40),
       P=st.integers(1, 700), rows=st.integers(1, 300))
def test_invariants_random(lens, P, rows):
    check_invariants(lens, P, rows, ref_schedule(lens, P, rows))


def test_invariants_at_config_shapes():
    rng = np.random.default_rng(0)
    cases = [
        ([64, 200], ref_num_parts(16, 256), 16),
        (rng.integers(1, 4097, 64).tolist(), ref_num_parts(128, 256), 128),
        ([4096] * 128, ref_num_parts(256, 256), 256),
        ([131072] * 8 + [1] * 8, ref_num_parts(64, 256), 64),
        ([2048] * 32, ref_num_parts(16, 256), 16),
        ([0] * 5, 3, 16),
        ([64 * 7], 1000, 16),
    ]
    for lens, P, rows in cases:
        check_invariants(lens, P, rows, ref_schedule(lens, P, rows))


def test_long_requests_get_many_splits():
    # the skewed long-context shape cuts long requests into more than 32 splits
    # (past the pages' one-warp combine fast path); a larger part count pushes
    # past one wavefront's 64 lanes
    u = unpack_schedule(ref_schedule([131072] * 8 + [100] * 8, ref_num_parts(64, 256), 64))
    assert u["max_splits"] > 32
    u = unpack_schedule(ref_schedule([131072] * 8 + [100] * 8, 1024, 64))
    assert u["max_splits"] > 64
