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

Swapping preempted sequences to host memory and back (inferensys glossary,
third and fifth paragraphs; crackai.dev "How It Works", preemption and
swapping), with these readings:
  * the swap space is a second pool of block ids with its own LIFO free
    list, first pops 0, 1, 2, ...;
  * a group swap moves the distinct blocks of the given sequences, taken in
    order of first appearance (sequences in the given order, each table in
    logical order); each gets one block of the other pool, holding as many
    references as the group makes to it;
  * the old blocks lose those references, and the ones left unreferenced
    are pushed back in reverse order of first appearance;
  * a swapped sequence keeps its length (generation resumes where it
    stopped) but cannot be forked, appended to or exported; freeing it
    releases its swap blocks.
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
        self.tables = {}   # seq_id -> list of physical blocks (swap blocks when swapped)
        self.lengths = {}  # seq_id -> tokens held
        self.swapped = {}  # seq_id -> True while its blocks live in the swap space
        self.host_free = []
        self.host_refcount = []

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
        self.swapped[seq_id] = False

    def fork(self, parent, child):
        if parent not in self.tables:
            raise AllocError(ERR_UNKNOWN_SEQ, "unknown parent %r" % (parent,))
        if child in self.tables:
            raise AllocError(ERR_INVALID_ARG, "child %r exists" % (child,))
        if self.swapped[parent]:
            raise AllocError(ERR_INVALID_ARG, "parent %r is swapped out" % (parent,))
        blocks = list(self.tables[parent])
        for b in blocks:
            self.refcount[b] += 1
        self.tables[child] = blocks
        self.lengths[child] = self.lengths[parent]
        self.swapped[child] = False

    def append_slot(self, seq_id):
        """Reserve the next position; returns (slot, cow_src, cow_dst), -1 when no copy."""
        if seq_id not in self.tables:
            raise AllocError(ERR_UNKNOWN_SEQ, "unknown sequence %r" % (seq_id,))
        if self.swapped[seq_id]:
            raise AllocError(ERR_INVALID_ARG, "sequence %r is swapped out" % (seq_id,))
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
        refs, free = ((self.host_refcount, self.host_free) if self.swapped[seq_id]
                      else (self.refcount, self.free))
        for b in reversed(self.tables[seq_id]):
            refs[b] -= 1
            if refs[b] == 0:
                free.append(b)
        del self.tables[seq_id]
        del self.lengths[seq_id]
        del self.swapped[seq_id]

    # --- swapping ----------------------------------------------------------
    def set_swap_space(self, num_host_blocks: int):
        if num_host_blocks < 0:
            raise AllocError(ERR_INVALID_ARG, "negative swap space")
        if any(self.swapped.values()):
            raise AllocError(ERR_INVALID_ARG, "a sequence is swapped out")
        self.host_free = list(range(num_host_blocks - 1, -1, -1))   # pops 0, 1, 2, ...
        self.host_refcount = [0] * num_host_blocks

    def swap_out(self, seq_ids):
        """Returns the (device block, swap block) pairs to copy."""
        return self._move(list(seq_ids), to_host=True)

    def swap_in(self, seq_ids):
        """Returns the (swap block, device block) pairs to copy."""
        return self._move(list(seq_ids), to_host=False)

    def _move(self, seq_ids, to_host):
        seen = set()
        for sid in seq_ids:
            if sid not in self.tables:
                raise AllocError(ERR_UNKNOWN_SEQ, "unknown sequence %r" % (sid,))
            if self.swapped[sid] == to_host:
                raise AllocError(ERR_INVALID_ARG, "sequence %r already there" % (sid,))
            if sid in seen:
                raise AllocError(ERR_INVALID_ARG, "sequence %r given twice" % (sid,))
            seen.add(sid)
        uses = {}   # block -> references from the group, in order of first appearance
        for sid in seq_ids:
            for b in self.tables[sid]:
                uses[b] = uses.get(b, 0) + 1
        if to_host:
            old_ref, old_free, new_ref, new_free = (self.refcount, self.free,
                                                    self.host_refcount, self.host_free)
        else:
            old_ref, old_free, new_ref, new_free = (self.host_refcount, self.host_free,
                                                    self.refcount, self.free)
        if len(uses) > len(new_free):
            raise AllocError(ERR_OUT_OF_BLOCKS, "target pool exhausted")
        where, pairs = {}, []
        for b, n in uses.items():
            t = new_free.pop()
            new_ref[t] = n
            where[b] = t
            pairs.append((b, t))
        for b in reversed(list(uses)):
            old_ref[b] -= uses[b]
            if old_ref[b] == 0:
                old_free.append(b)
        for sid in seq_ids:
            self.tables[sid] = [where[b] for b in self.tables[sid]]
            self.swapped[sid] = to_host
        return pairs

    # --- invariants --------------------------------------------------------
    def check_invariants(self):
        refs = [0] * self.num_blocks
        host_refs = [0] * len(self.host_refcount)
        for sid, tab in self.tables.items():
            for b in tab:
                if self.swapped[sid]:
                    host_refs[b] += 1
                else:
                    refs[b] += 1
        assert refs == self.refcount, "refcounts disagree with the tables"
        assert host_refs == self.host_refcount, "swap refcounts disagree with the tables"
        free = set(self.free)
        assert len(free) == len(self.free), "a block is on the free list twice"
        for b in range(self.num_blocks):
            assert (b in free) == (self.refcount[b] == 0), "block %d free/referenced mismatch" % b
        hfree = set(self.host_free)
        assert len(hfree) == len(self.host_free), "a swap block is on its free list twice"
        for b in range(len(self.host_refcount)):
            assert (b in hfree) == (self.host_refcount[b] == 0), "swap block %d mismatch" % b
        for sid, tab in self.tables.items():
            L = self.lengths[sid]
            assert len(tab) == -(-L // self.block_size), "table length disagrees with tokens"
            assert len(tab) * self.block_size - L < self.block_size or L == 0
