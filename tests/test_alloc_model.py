"""Pins of the Python allocator model (the allocator's oracle).

* the pages' worked example: ten users sharing a 4,000-token prompt hold the
  prompt's 250 blocks once, new 16-token blocks come on demand, and a
  finished request's blocks are the very next ones handed out;
* internal fragmentation below one block per sequence;
* invariants after every operation of random traces;
* hand traces of copy-on-write and of all-or-nothing failure.
"""
import json
import os

import numpy as np
import pytest

from oracle.alloc_model import (AllocError, BlockAllocatorModel, ERR_INVALID_ARG,
                                ERR_OUT_OF_BLOCKS, ERR_UNKNOWN_SEQ)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "shared_prompt_worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_example_prompt_is_stored_once():
    g = _golden()
    users = g["printed"]["users"]
    P = g["printed"]["system_prompt_tokens"]
    Bs = g["printed"]["block_size_tokens"]
    a = BlockAllocatorModel(4096, Bs)
    a.create(0, P)
    for u in range(1, users):
        a.fork(0, u)
    distinct = {b for u in range(users) for b in a.table(u)}
    assert len(distinct) == g["derived"]["prompt_blocks_shared"] == 250
    assert sum(len(a.table(u)) for u in range(users)) == g["derived"]["prompt_blocks_without_sharing"]
    assert all(a.refcount[b] == users for b in distinct)
    a.check_invariants()


def test_worked_example_on_demand_blocks_and_immediate_reuse():
    g = _golden()
    users, P, Bs = 10, g["printed"]["system_prompt_tokens"], g["printed"]["block_size_tokens"]
    a = BlockAllocatorModel(4096, Bs)
    a.create(0, P)
    for u in range(1, users):
        a.fork(0, u)
    # The prompt ends on a block boundary: each user's first generated token
    # pops a fresh private block, no copy.
    for k in range(1, 40):
        for u in range(users):
            slot, src, dst = a.append_slot(u)
            assert src == dst == -1
        distinct = {b for u in range(users) for b in a.table(u)}
        assert len(distinct) == 250 + users * (-(-k // Bs))
        a.check_invariants()
    # User 3 finishes: its private blocks return, and the next request gets
    # exactly those blocks, first logical block first.
    private = a.table(3)[250:]
    a.free_seq(3)
    assert a.num_free() == 4096 - 250 - (users - 1) * len(private) - 0
    a.create(100, 3 * Bs)
    assert a.table(100) == private[:3]
    a.check_invariants()


def test_waste_is_below_one_block_per_sequence():
    rng = np.random.default_rng(41)
    for Bs in (8, 16, 32, 64):
        a = BlockAllocatorModel(100000, Bs)
        lens = rng.integers(1, 5000, size=200)
        for i, L in enumerate(lens):
            a.create(i, int(L))
        for i, L in enumerate(lens):
            waste = len(a.table(i)) * Bs - L
            assert 0 <= waste <= Bs - 1
        a.check_invariants()


def test_default_and_given_pop_order():
    a = BlockAllocatorModel(6, 4)
    a.create("s", 9)
    assert a.table("s") == [0, 1, 2]
    b = BlockAllocatorModel(6, 4, initial_free_order=[5, 3, 1, 0, 2, 4])
    b.create("s", 9)
    b.create("t", 1)
    assert b.table("s") == [5, 3, 1] and b.table("t") == [0]


def test_free_returns_first_block_first():
    a = BlockAllocatorModel(8, 4)
    a.create(1, 12)                  # blocks 0,1,2
    a.free_seq(1)
    a.create(2, 4)
    assert a.table(2) == [0]
    a.create(3, 8)
    assert a.table(3) == [1, 2]


def test_copy_on_write_fires_only_on_a_shared_partial_block():
    a = BlockAllocatorModel(10, 4)
    a.create("p", 6)                 # blocks 0,1; last block holds 2 of 4
    a.fork("p", "c")
    assert a.refcount[:2] == [2, 2]
    slot, src, dst = a.append_slot("c")
    assert (src, dst) == (1, 2) and slot == 2 * 4 + 2
    assert a.table("c") == [0, 2] and a.table("p") == [0, 1]
    assert a.refcount[:3] == [2, 1, 1]
    # The parent is now the last owner of block 1: it writes in place.
    slot, src, dst = a.append_slot("p")
    assert (src, dst) == (-1, -1) and slot == 1 * 4 + 2
    a.check_invariants()


def test_full_shared_block_is_never_copied():
    a = BlockAllocatorModel(10, 4)
    a.create("p", 8)                 # two full blocks
    a.fork("p", "c")
    slot, src, dst = a.append_slot("c")
    assert (src, dst) == (-1, -1)
    assert a.table("c") == [0, 1, 2] and slot == 8
    assert a.refcount[:3] == [2, 2, 1]


def test_failures_leave_state_unchanged():
    a = BlockAllocatorModel(3, 4)
    a.create(0, 6)
    a.fork(0, 1)
    snap = (list(a.free), list(a.refcount), {k: list(v) for k, v in a.tables.items()}, dict(a.lengths))
    cases = [
        (lambda: a.create(2, 9), ERR_OUT_OF_BLOCKS),
        (lambda: a.create(0, 1), ERR_INVALID_ARG),
        (lambda: a.fork(7, 8), ERR_UNKNOWN_SEQ),
        (lambda: a.fork(0, 1), ERR_INVALID_ARG),
        (lambda: a.free_seq(9), ERR_UNKNOWN_SEQ),
        (lambda: a.append_slot(9), ERR_UNKNOWN_SEQ),
    ]
    for fn, code in cases:
        with pytest.raises(AllocError) as e:
            fn()
        assert e.value.code == code
        assert snap == (list(a.free), list(a.refcount), {k: list(v) for k, v in a.tables.items()},
                        dict(a.lengths))
    # One free block left: the first CoW succeeds, the second runs out.
    a.append_slot(1)
    a.fork(0, 2)
    snap = (list(a.free), list(a.refcount), {k: list(v) for k, v in a.tables.items()}, dict(a.lengths))
    with pytest.raises(AllocError) as e:
        a.append_slot(2)
    assert e.value.code == ERR_OUT_OF_BLOCKS
    assert snap == (list(a.free), list(a.refcount), {k: list(v) for k, v in a.tables.items()},
                    dict(a.lengths))


def random_trace(seed, n_ops=400, num_blocks=64, block_size=4):
    """A seeded op list over create/fork/append/free and group swaps out and
    in (also used against the C++ allocator).  Ops on swapped or unknown
    sequences are included on purpose: they must fail the same way."""
    rng = np.random.default_rng(seed)
    ops, live, next_id = [("swap_space", num_blocks // 2)], [], 0
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.18 or not live:
            ops.append(("create", next_id, int(rng.integers(0, 3 * block_size + 1))))
            live.append(next_id); next_id += 1
        elif r < 0.32:
            ops.append(("fork", int(rng.choice(live)), next_id))
            live.append(next_id); next_id += 1
        elif r < 0.76:
            ops.append(("append", int(rng.choice(live))))
        elif r < 0.86:
            s = int(rng.choice(live)); live.remove(s)
            ops.append(("free", s))
        else:
            k = int(rng.integers(1, min(4, len(live)) + 1))
            group = [int(x) for x in rng.choice(live, size=k, replace=False)]
            ops.append(("swap_out" if rng.random() < 0.5 else "swap_in", group))
        if rng.random() < 0.03:
            ops.append(("free", 10 ** 6))           # unknown id
    return ops


def apply_model(a, op):
    try:
        if op[0] == "create":
            a.create(op[1], op[2]); return (0,)
        if op[0] == "fork":
            a.fork(op[1], op[2]); return (0,)
        if op[0] == "append":
            return (0,) + a.append_slot(op[1])
        if op[0] == "swap_space":
            a.set_swap_space(op[1]); return (0,)
        if op[0] == "swap_out":
            return (0, tuple(a.swap_out(op[1])))
        if op[0] == "swap_in":
            return (0, tuple(a.swap_in(op[1])))
        a.free_seq(op[1]); return (0,)
    except AllocError as e:
        return (e.code,)


@pytest.mark.parametrize("seed", range(6))
def test_invariants_hold_after_every_operation(seed):
    a = BlockAllocatorModel(64, 4, initial_free_order=np.random.default_rng(seed).permutation(64))
    live = set()
    for op in random_trace(seed):
        r = apply_model(a, op)
        a.check_invariants()
        if op[0] in ("swap_out", "swap_in") and r[0] == 0:
            # Every moved block went to a distinct block of the other pool.
            dsts = [t for _, t in r[1]]
            assert len(set(dsts)) == len(dsts)
            assert all(a.swapped[sid] == (op[0] == "swap_out") for sid in op[1])
        if op[0] == "append" and r[0] == 0:
            slot, src, dst = r[1:]
            # After an append the written block belongs to this sequence alone.
            assert a.refcount[a.table(op[1])[-1]] == 1
            assert slot // 4 == a.table(op[1])[-1]
            assert (src == -1) == (dst == -1)


# ---- swapping (inferensys glossary, third and fifth paragraphs) -------------

def _group():
    """Prompt 0 of 10 tokens (3 blocks of 4), child 1 forked from it and
    grown by 3 tokens (copy of the shared partial block, then a new block)."""
    a = BlockAllocatorModel(16, 4)
    a.set_swap_space(8)
    a.create(0, 10)
    a.fork(0, 1)
    for _ in range(3):
        a.append_slot(1)
    return a


def test_swapping_a_group_moves_each_distinct_block_once():
    a = _group()
    assert a.table(0) == [0, 1, 2] and a.table(1) == [0, 1, 3, 4]
    pairs = a.swap_out([0, 1])
    # Distinct blocks in first-appearance order, swap blocks popped 0, 1, 2, ...
    assert pairs == [(0, 0), (1, 1), (2, 2), (3, 3), (4, 4)]
    assert a.host_refcount[:5] == [2, 2, 1, 1, 1]
    assert a.table(0) == [0, 1, 2] and a.table(1) == [0, 1, 3, 4]     # now swap-space ids
    assert a.num_free() == 16 and all(r == 0 for r in a.refcount)
    # Freed in reverse order of first appearance: block 0 is handed out next.
    assert a.free[-5:] == [4, 3, 2, 1, 0]
    a.check_invariants()


def test_a_sharer_left_behind_keeps_the_original():
    a = _group()
    pairs = a.swap_out([1])
    assert [b for b, _ in pairs] == [0, 1, 3, 4]
    assert a.refcount[0] == 1 and a.refcount[1] == 1      # still held by sequence 0
    assert a.refcount[3] == 0 and a.refcount[4] == 0
    a.check_invariants()


def test_swap_round_trip_resumes_where_it_stopped():
    a = _group()
    lens = (a.length(0), a.length(1))
    a.swap_out([0, 1])
    a.create(5, 12)                                       # someone else takes the blocks
    pairs = a.swap_in([1, 0])
    assert (a.length(0), a.length(1)) == lens
    # Sharing inside the group survives: the two prefixes are one set of blocks.
    assert a.table(0)[:2] == a.table(1)[:2]
    assert a.refcount[a.table(0)[0]] == 2
    assert sorted(a.table(0) + a.table(1)[2:]) == sorted(t for _, t in pairs)
    slot, src, dst = a.append_slot(1)                     # next position, same offset rule
    assert slot % 4 == lens[1] % 4 and src == -1
    a.check_invariants()


def test_swapped_sequences_refuse_growth_and_failed_swaps_change_nothing():
    a = _group()
    a.swap_out([1])
    for fn, code in [(lambda: a.append_slot(1), ERR_INVALID_ARG),
                     (lambda: a.fork(1, 9), ERR_INVALID_ARG),
                     (lambda: a.swap_out([1]), ERR_INVALID_ARG),
                     (lambda: a.swap_in([0]), ERR_INVALID_ARG),
                     (lambda: a.swap_out([0, 0]), ERR_INVALID_ARG),
                     (lambda: a.swap_in([7]), ERR_UNKNOWN_SEQ),
                     (lambda: a.set_swap_space(4), ERR_INVALID_ARG)]:
        snap = (list(a.free), list(a.refcount), list(a.host_free), list(a.host_refcount),
                {k: list(v) for k, v in a.tables.items()}, dict(a.swapped))
        with pytest.raises(AllocError) as e:
            fn()
        assert e.value.code == code
        assert snap == (list(a.free), list(a.refcount), list(a.host_free),
                        list(a.host_refcount), {k: list(v) for k, v in a.tables.items()},
                        dict(a.swapped))
    # The swap space has 4 free blocks left; sequence 0's 3 fit, a bigger group does not.
    a.create(3, 16)
    with pytest.raises(AllocError) as e:
        a.swap_out([0, 3])
    assert e.value.code == ERR_OUT_OF_BLOCKS
    a.free_seq(1)                                         # releases its swap blocks
    assert a.host_refcount == [0] * 8 and len(a.host_free) == 8
    a.check_invariants()
