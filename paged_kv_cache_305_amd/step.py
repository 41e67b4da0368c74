"""One decode step of a paged KV cache, as a serving loop would run it.

Host: the block allocator reserves each sequence's next slot, allocating a
block at a block boundary and returning a (src, dst) copy pair when the
last block is shared (copy-on-write).  Device, in stream order: copy_blocks
on the pairs, then the attention over every sequence's cached tokens with
the new tokens written into their slots by the same launch
(paged_attention_decode_append, or paged_attention_decode_prefix when the
sequences share a prefix) -- or, unfused, reshape_and_cache followed by the
attention.  Both give the same pools and outputs.

The host part runs once when the step is built; ``run()`` only launches the
kernels, so it can be repeated (same pairs, same slots, same reads) for
timing.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import _binding as B


@dataclass
class DecodeStep:
    query: object            # [B, Hq, d]
    key_cache: object
    value_cache: object
    new_key: object          # [B, Hkv, d]
    new_value: object
    slot_mapping: object     # int64 [B]
    cow_pairs: object        # int64 [n, 2] (n may be 0)
    block_tables: object     # int32 [B, max_blocks]
    context_lens: object     # int32 [B]
    out: object              # [B, Hq, d]
    workspace: Optional[object]
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_context_len: int
    scale: float
    partition_size: int
    kv_reused: bool = False
    # Write the new tokens from inside the attention launch (True or None,
    # the default) or with reshape_and_cache first (False).
    fused: Optional[bool] = None
    # Tokens every sequence shares in the same blocks (0: none); when set,
    # the attention reads them once for all sequences.
    prefix_len: int = 0
    # Copy-on-write sources per sequence (int64 [B], -1: none) when every
    # copy pair is a sequence's new-token block, else None.
    cow_src: Optional[object] = None
    # With the in-launch write, copy the pairs inside the attention launch
    # too (True or None, the default, when cow_src exists) or with
    # copy_blocks first (False).
    cow_fused: Optional[bool] = None

    @property
    def num_pairs(self) -> int:
        return int(self.cow_pairs.shape[0])

    def copy(self, stream=None):
        if self.num_pairs:
            B.copy_blocks(self.key_cache, self.value_cache, self.cow_pairs,
                          num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
                          block_size=self.block_size, num_blocks=self.num_blocks, stream=stream)

    def write(self, stream=None):
        B.reshape_and_cache(self.new_key, self.new_value, self.key_cache, self.value_cache,
                            self.slot_mapping, block_size=self.block_size,
                            num_blocks=self.num_blocks, stream=stream)

    def use_prefix(self, prefix_len: int):
        """Attend with the shared-prefix kernel from now on (sizing its
        workspace)."""
        import torch
        self.prefix_len = int(prefix_len)
        if self.prefix_len:
            nseq, hq, d = self.query.shape
            nbytes = B.paged_attention_prefix_workspace_bytes(
                nseq, hq, self.num_kv_heads, d, self.max_context_len, self.prefix_len,
                self.query.dtype)
            self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8,
                                         device=self.query.device)
        return self

    def attend(self, stream=None, append=False, cow=False):
        extra = dict(new_key=self.new_key, new_value=self.new_value,
                     slot_mapping=self.slot_mapping) if append else {}
        if cow:
            extra["cow_src"] = self.cow_src
        if self.prefix_len:
            B.paged_attention_decode_prefix(
                self.out, self.query, self.key_cache, self.value_cache, self.block_tables,
                self.context_lens, prefix_len=self.prefix_len, num_kv_heads=self.num_kv_heads,
                block_size=self.block_size, max_context_len=self.max_context_len,
                scale=self.scale, workspace=self.workspace, num_blocks=self.num_blocks,
                stream=stream, **extra)
            return
        B.paged_attention_decode(self.out, self.query, self.key_cache, self.value_cache,
                                 self.block_tables, self.context_lens,
                                 num_kv_heads=self.num_kv_heads, block_size=self.block_size,
                                 max_context_len=self.max_context_len, scale=self.scale,
                                 partition_size=self.partition_size, workspace=self.workspace,
                                 num_blocks=self.num_blocks, kv_reused=self.kv_reused,
                                 stream=stream, **extra)

    # The in-launch write stores the new tokens after each wave's reads; on
    # MI355X that costs less than a separate reshape_and_cache pass and its
    # launch at every batch size measured, so it is the default.

    @property
    def uses_fused_write(self) -> bool:
        return True if self.fused is None else self.fused

    @property
    def uses_fused_copy(self) -> bool:
        """Copy-on-write inside the attention launch: with the in-launch
        write, when there are pairs and each is a sequence's new-token
        block."""
        return (self.uses_fused_write and self.num_pairs > 0 and self.cow_src is not None
                and self.cow_fused is not False)

    def capture(self):
        """Record run() into a HIP graph (torch.cuda.CUDAGraph); replay()
        then repeats the step's launches with one call.  The graph reads
        and writes the step's tensors in place: refill them (copy_) to run
        the step on new inputs."""
        import torch
        side = torch.cuda.Stream()             # default priority
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()                         # settle lazy set-up outside the capture
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        self._graph = g
        return g

    def replay(self):
        self._graph.replay()
        return self.out

    def run(self, stream=None):
        """One launch that copies the shared blocks, writes the new tokens and
        attends (fused); or copy_blocks first, then that launch without the
        copies; or copy_blocks, reshape_and_cache and attention."""
        if self.uses_fused_copy:
            self.attend(stream, append=True, cow=True)
            return self.out
        self.copy(stream)
        if self.uses_fused_write:
            self.attend(stream, append=True)
        else:
            self.write(stream)
            self.attend(stream)
        return self.out


def _finish(query, key_cache, value_cache, new_key, new_value, slots, pairs, tables, lens, *,
            num_kv_heads, head_dim, block_size, num_blocks, scale, partition_size,
            out_dtype=None) -> DecodeStep:
    import torch
    dev = query.device
    t_slots = torch.as_tensor(np.ascontiguousarray(slots, dtype=np.int64)).to(dev)
    t_pairs = torch.as_tensor(np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)).to(dev)
    t_tab = torch.as_tensor(np.ascontiguousarray(tables, dtype=np.int32)).to(dev)
    t_lens = torch.as_tensor(np.ascontiguousarray(lens, dtype=np.int32)).to(dev)
    mcl = int(np.max(lens)) if len(lens) else 0
    out = torch.empty(query.shape, dtype=out_dtype or query.dtype, device=dev)
    nbytes = B.paged_attention_workspace_bytes(query.shape[0], query.shape[1], num_kv_heads,
                                               head_dim, mcl, partition_size, query.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    step = DecodeStep(query, key_cache, value_cache, new_key, new_value, t_slots, t_pairs, t_tab,
                      t_lens, out, ws, num_kv_heads, head_dim, block_size, num_blocks, mcl, scale,
                      partition_size)
    step.cow_src = _cow_sources(slots, pairs, block_size, dev)
    return step


def _cow_sources(slots, pairs, block_size, dev):
    """Per-sequence copy sources (int64 [B], -1: none) when every pair's
    destination is exactly one sequence's new-token block, else None."""
    import torch
    slots = np.asarray(slots, dtype=np.int64)
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if pairs.shape[0] == 0:
        return None
    src = np.full(slots.shape[0], -1, np.int64)
    seq_of_block = {}
    for i, sl in enumerate(slots):
        if sl >= 0:
            seq_of_block.setdefault(int(sl) // block_size, []).append(i)
    for s_blk, d_blk in pairs:
        owners = seq_of_block.get(int(d_blk), [])
        if len(owners) != 1 or src[owners[0]] >= 0:
            return None
        src[owners[0]] = s_blk
    return torch.as_tensor(src).to(dev)


def step_from_case(case, partition_size: int, out_dtype=None) -> DecodeStep:
    """A step over a workload whose tables are given: write the token at
    position L-1 of each sequence, then attend over all L tokens."""
    return _finish(case.query, case.key_cache, case.value_cache, case.new_key, case.new_value,
                   case.slot_mapping, np.zeros((0, 2), np.int64), case.block_tables,
                   case.context_lens, num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                   block_size=case.block_size, num_blocks=case.num_blocks, scale=case.scale,
                   partition_size=partition_size, out_dtype=out_dtype)


SHADOW = 1 << 40   # shadow sequence ids: seq_id + SHADOW


def build_shared_prefix_state(plan) -> "B.BlockAllocator":
    """Allocator state before the step: one prompt, batch-1 forks, private tails."""
    a = B.BlockAllocator(plan.num_blocks, plan.block_size, plan.perm)
    a.create(0, int(plan.prompt))
    for i in range(1, plan.batch):
        a.fork(0, i)
    for i in range(plan.batch):
        for _ in range(int(plan.tails[i])):
            a.append_slot(i)
    return a


def shared_prefix_step(plan, tensors, partition_size: int, out_dtype=None, prefix=False):
    """The shared-prefix sampling step: fork every sequence into a shadow
    that shares all its blocks (beam-search style), append one token to each
    sequence in ascending id (copy-on-write where the last block is partial
    and shared), then free the shadows.  With prefix=True the attention
    reads the prompt's full blocks once for all sequences.  Returns (step,
    host record)."""
    a = build_shared_prefix_state(plan)
    for i in range(plan.batch):
        a.fork(i, SHADOW + i)
    slots = np.empty(plan.batch, np.int64)
    pairs = []
    for i in range(plan.batch):
        s, src, dst = a.append_slot(i)
        slots[i] = s
        if src >= 0:
            pairs.append((src, dst))
    for i in range(plan.batch):
        a.free(SHADOW + i)
    lens = np.array([a.seq_len(i) for i in range(plan.batch)], np.int64)
    max_blocks = int(-(-lens.max() // plan.block_size))
    tables, lens32 = a.build_block_tables(list(range(plan.batch)), max_blocks)
    pairs = np.array(pairs, np.int64).reshape(-1, 2)
    step = _finish(tensors["query"], tensors["key_cache"], tensors["value_cache"],
                   tensors["new_key"], tensors["new_value"], slots, pairs, tables, lens32,
                   num_kv_heads=tensors["num_kv_heads"], head_dim=tensors["head_dim"],
                   block_size=plan.block_size, num_blocks=plan.num_blocks,
                   scale=tensors["scale"], partition_size=partition_size, out_dtype=out_dtype)
    # The prompt's blocks are shared by every sequence: keep them in the caches.
    step.kv_reused = True
    if prefix:
        step.use_prefix(plan.prompt // plan.block_size * plan.block_size)
    record = dict(slots=slots, pairs=pairs, tables=tables, lens=lens32, allocator=a)
    return step, record
