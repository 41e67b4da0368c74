"""Plain Python model of the paged KV block allocator -- TEST INFRASTRUCTURE ONLY.

Follows the memory-management operations the pages state:
  * fixed-size blocks, a per-sequence table of logical -> physical block
    (dmarx note-023, Method; crackai.dev "How It Works", block table);
  * a block is taken only when a sequence's growth needs one, never
    reserved up front for a maximum length (note-023 Method; crackai.dev,
    on-demand allocation);
  * blocks freed when a sequence finishes and reused right away
    (note-023 Method; skillsintelligence glossary, worked example);
  * physical blocks shared by reference between sequences with a common
    prefix, and copied only when one sharer writes (note-023 Concepts
    "Copy-on-write"; inferensys glossary, second paragraph; crackai.dev,
    copy-on-write sharing).

Where the pages leave the policy open, this model takes these readings:
  * the free list is a LIFO stack; by default the first pops are 0, 1, 2, ...
    or, when an initial order is given, order[0], order[1], ...;
  * a sequence's blocks are pushed back from its last logical block to its
    first, so its first block is the next one popped;
  * a copy fires only when appending into a partially filled last block
    that is shared (refcount > 1); a full shared block is never copied, the
    append pops a fresh block instead;
  * every operation is all-or-nothing: on pool exhaustion or a bad id the
    state is unchanged.
"""
from __future__ import annotations

OK = 0
ERR_INVALID_ARG = -1
ERR_OUT_OF_BLOCKS = -3
ERR_UNKNOWN_SEQ = -4


class AllocError(Exception):
    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


class BlockAllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError(ERR_INVALID_ARG, "num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError(ERR_INVALID_ARG, "initial order must be a permutation of the pool")
        self.num_blocks = num_blocks
        self.block_size = block_size
        # Top of the stack is the end of the list: pops come out as order[0], order[1], ...
        self.free = list(reversed(order))
        self.refcount = [0] * num_blocks
        self.tables = {}   # seq_id -> list of physical blocks
        self.lengths = {}  # seq_id -> tokens held

    # --- queries -----------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def table(self, seq_id):
        if seq_id not in self.tables:
            raise AllocError(ERR_UNKNOWN_SEQ, "unknown sequence %r" % (seq_id,))
        return list(self.tables[seq_id])

    def length(self, seq_id) -> int:
        if seq_id not in self.lengths:
            raise AllocError(ERR_UNKNOWN_SEQ, "unknown sequence %r" % (seq_id,))
        return self.lengths[seq_id]

    # --- operations --------------------------------------------------------
    def create(self, seq_id, num_tokens: int):
        if seq_id in self.tables:
            raise AllocError(ERR_INVALID_ARG, "sequence %r exists" % (seq_id,))
        if num_tokens < 0:
            raise AllocError(ERR_INVALID_ARG, "negative length")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise AllocError(ERR_OUT_OF_BLOCKS, "pool exhausted")
        blocks = [self.free.pop() for _ in range(need)]
        for b in blocks:
            self.refcount[b] = 1
        self.tables[seq_id] = blocks
        self.lengths[seq_id] = num_tokens

    def fork(self, parent, child):
        if parent not in self.tables:
            raise AllocError(ERR_UNKNOWN_SEQ, "unknown parent %r" % (parent,))
        if child in self.tables:
            raise AllocError(ERR_INVALID_ARG, "child %r exists" % (child,))
        blocks = list(self.tables[parent])
        for b in blocks:
            self.refcount[b] += 1
        self.tables[child] = blocks
        self.lengths[child] = self.lengths[parent]

    def append_slot(self, seq_id):
        """Reserve the next position; returns (slot, cow_src, cow_dst), -1 when no copy."""
        if seq_id not in self.tables:
            raise AllocError(ERR_UNKNOWN_SEQ, "unknown sequence %r" % (seq_id,))
        tab = self.tables[seq_id]
        pos = self.lengths[seq_id]
        off = pos % self.block_size
        src = dst = -1
        if off == 0:
            if not self.free:
                raise AllocError(ERR_OUT_OF_BLOCKS, "pool exhausted")
            b = self.free.pop()
            self.refcount[b] = 1
            tab.append(b)
        else:
            last = tab[-1]
            if self.refcount[last] > 1:
                if not self.free:
                    raise AllocError(ERR_OUT_OF_BLOCKS, "pool exhausted")
                b = self.free.pop()
                self.refcount[b] = 1
                self.refcount[last] -= 1
                tab[-1] = b
                src, dst = last, b
        self.lengths[seq_id] = pos + 1
        return tab[-1] * self.block_size + off, src, dst

    def free_seq(self, seq_id):
        if seq_id not in self.tables:
            raise AllocError(ERR_UNKNOWN_SEQ, "unknown sequence %r" % (seq_id,))
        for b in reversed(self.tables[seq_id]):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.tables[seq_id]
        del self.lengths[seq_id]

    # --- invariants --------------------------------------------------------
    def check_invariants(self):
        refs = [0] * self.num_blocks
        for tab in self.tables.values():
            for b in tab:
                refs[b] += 1
        assert refs == self.refcount, "refcounts disagree with the tables"
        free = set(self.free)
        assert len(free) == len(self.free), "a block is on the free list twice"
        for b in range(self.num_blocks):
            assert (b in free) == (self.refcount[b] == 0), "block %d free/referenced mismatch" % b
        for sid, tab in self.tables.items():
            L = self.lengths[sid]
            assert len(tab) == -(-L // self.block_size), "table length disagrees with tokens"
            assert len(tab) * self.block_size - L < self.block_size or L == 0
