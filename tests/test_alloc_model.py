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

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "shared_prompt_l138.json")


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
    """A seeded op list over create/fork/append/free (also used against the C++ allocator)."""
    rng = np.random.default_rng(seed)
    ops, live, next_id = [], [], 0
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.2 or not live:
            ops.append(("create", next_id, int(rng.integers(0, 3 * block_size + 1))))
            live.append(next_id); next_id += 1
        elif r < 0.35:
            ops.append(("fork", int(rng.choice(live)), next_id))
            live.append(next_id); next_id += 1
        elif r < 0.85:
            ops.append(("append", int(rng.choice(live))))
        else:
            s = int(rng.choice(live)); live.remove(s)
            ops.append(("free", s))
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
        if op[0] == "append" and r[0] == 0:
            slot, src, dst = r[1:]
            # After an append the written block belongs to this sequence alone.
            assert a.refcount[a.table(op[1])[-1]] == 1
            assert slot // 4 == a.table(op[1])[-1]
            assert (src == -1) == (dst == -1)
