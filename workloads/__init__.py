"""Seeded synthetic inputs for the paged decode path.

This module holds no attention arithmetic and imports neither the HIP
binding nor the CPU oracle.  It produces only what both sides consume:
shapes, seeded random draws, and the integer structure of a paged KV cache
(context lengths, a random permutation of the physical block pool, the
per-sequence block tables that take consecutive runs of that permutation,
and the slot of each new token).

Pool tensors are returned layout-agnostic as ``[num_blocks, num_kv_heads,
block_size * head_dim]``: every (block, KV head) chunk is one contiguous run
of ``block_size * head_dim`` elements, filled i.i.d. N(0, 1).  How the
elements of a chunk map to (token, feature) is the library's layout and is
not needed to draw i.i.d. values.

Seeding: config k (0-based, in the order of ``CONFIG_ORDER``) uses
``seed = 305 + k``.  Integer structure comes from
``numpy.random.default_rng(seed)`` in the order lengths -> pool permutation
(-> tails for the shared-prefix workload); float tensors come from a
``torch.Generator`` on the target device seeded with the same value, drawn
in the order q -> key pool -> value pool -> new key -> new value, as fp32
N(0, 1) and narrowed round-to-nearest-even to bf16 where the workload is
bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

CONFIG_ORDER = ("tiny", "7b", "70b", "shared", "long")
# Workloads beyond the five, seeded after them in this order.
EXTRA_ORDER = ("mixed",)

# Workload shapes.  "lens" fixes the lengths; "len_range" draws them
# uniformly (inclusive).  pool: "1.5x" = ceil(1.5 * blocks needed),
# "exact" = blocks needed, an int = that many blocks.
CONFIGS = {
    # 4 sequences, context {17,33,64,100}, 8 q = 8 KV heads, d 64, Bs 16,
    # fp32, 64-block pool, scale 1/sqrt(64).
    "tiny": dict(batch=4, lens=(17, 33, 64, 100), num_q_heads=8, num_kv_heads=8,
                 head_dim=64, block_size=16, dtype="fp32", pool=64),
    # Llama-2-7B-shaped single layer: batch 64, 32/32 heads, d 128, bf16,
    # Bs 16, context U[512, 2048], pool 1.5x the blocks needed.
    "7b": dict(batch=64, len_range=(512, 2048), num_q_heads=32, num_kv_heads=32,
               head_dim=128, block_size=16, dtype="bf16", pool="1.5x"),
    # 70B-shaped GQA: batch 256, 64 q / 8 KV heads, d 128, bf16, Bs 16,
    # context U[128, 4096], exactly the blocks needed, fully permuted.
    "70b": dict(batch=256, len_range=(128, 4096), num_q_heads=64, num_kv_heads=8,
                head_dim=128, block_size=16, dtype="bf16", pool="exact"),
    # Shared-prefix parallel sampling: 64 sequences forked from one
    # 4000-token prompt, private tails U[0, 512], 32 q / 8 KV heads.
    "shared": dict(batch=64, prompt=4000, tail_range=(0, 512), num_q_heads=32,
                   num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                   pool="1.5x"),
    # Long-context split-K: batch 8, context 32768, 32 q / 8 KV heads,
    # Bs 16 or 32, partitions of 512 tokens.
    "long": dict(batch=8, lens=(32768,) * 8, num_q_heads=32, num_kv_heads=8,
                 head_dim=128, block_size=16, dtype="bf16", pool="exact",
                 partition_size=512),
    # The 70B shape with one long context in the batch (continuous batching
    # of one long request among short ones): 255 contexts U[128, 4096] and
    # one of 131072 at a seeded position.
    "mixed": dict(batch=256, len_range=(128, 4096), long_len=131072, num_q_heads=64,
                  num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16", pool="exact"),
}

TORCH_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


def seed_for(name: str) -> int:
    if name in EXTRA_ORDER:
        return 305 + len(CONFIG_ORDER) + EXTRA_ORDER.index(name)
    return 305 + CONFIG_ORDER.index(name)


def blocks_for(length: int, block_size: int) -> int:
    return -(-int(length) // int(block_size))


@dataclass
class DecodeCase:
    """One decode step's inputs, all tensors on ``device``."""
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    num_blocks: int
    scale: float
    context_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray          # int32 [B, max_blocks]
    perm: np.ndarray                  # int32 [num_blocks] physical pop order
    query: torch.Tensor               # [B, Hq, d]
    key_cache: torch.Tensor           # [N, Hkv, Bs*d]
    value_cache: torch.Tensor         # [N, Hkv, Bs*d]
    new_key: Optional[torch.Tensor] = None     # [B, Hkv, d]
    new_value: Optional[torch.Tensor] = None   # [B, Hkv, d]
    slot_mapping: Optional[np.ndarray] = None  # int64 [B]
    partition_size: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0

    @property
    def torch_dtype(self) -> torch.dtype:
        return TORCH_DTYPES[self.dtype]


def _randn(gen: torch.Generator, shape, device, dtype: str) -> torch.Tensor:
    t = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    return t if dtype == "fp32" else t.to(torch.bfloat16)


def _pool(gen, num_blocks, hkv, chunk, device, dtype, chunk_rows=4096):
    """Draw a [num_blocks, hkv, chunk] pool in row chunks (bounded fp32 temp)."""
    out = torch.empty(num_blocks, hkv, chunk, device=device, dtype=TORCH_DTYPES[dtype])
    for s in range(0, num_blocks, chunk_rows):
        e = min(num_blocks, s + chunk_rows)
        out[s:e] = _randn(gen, (e - s, hkv, chunk), device, dtype)
    return out


def tables_from_perm(lengths, perm, block_size, max_blocks=None, pad=0):
    """Sequences take consecutive runs of ``perm`` in sequence order."""
    nb = [blocks_for(l, block_size) for l in lengths]
    width = max(1, max(nb) if nb else 1) if max_blocks is None else max_blocks
    tab = np.full((len(lengths), width), pad, dtype=np.int32)
    pos = 0
    for i, n in enumerate(nb):
        tab[i, :n] = perm[pos:pos + n]
        pos += n
    return tab


def slots_at(lengths, tables, block_size):
    """Slot of the token at position L-1 of each sequence (block*Bs + offset)."""
    s = np.empty(len(lengths), dtype=np.int64)
    for i, l in enumerate(lengths):
        p = int(l) - 1
        s[i] = int(tables[i, p // block_size]) * block_size + p % block_size if l > 0 else -1
    return s


@dataclass
class CaseStructure:
    """Integer structure of a decode workload (no tensors)."""
    name: str
    seed: int
    block_size: int
    lengths: np.ndarray     # int64 [B]
    num_blocks: int
    perm: np.ndarray        # int32 [num_blocks]
    tables: np.ndarray      # int32 [B, max blocks]
    slots: np.ndarray       # int64 [B], slot of position L-1


def case_structure(name: str, *, batch: Optional[int] = None, seed: Optional[int] = None,
                   block_size: Optional[int] = None, lens=None, len_range=None,
                   pool=None) -> CaseStructure:
    """Seeded lengths, pool permutation, tables and new-token slots of ``name``."""
    cfg = dict(CONFIGS[name])
    if name == "shared":
        raise ValueError("use shared_plan for the shared-prefix workload")
    seed = seed_for(name) if seed is None else seed
    bs = block_size or cfg["block_size"]
    rng = np.random.default_rng(seed)
    if lens is not None:
        lengths = np.asarray(lens, dtype=np.int64)
    elif len_range is not None or "len_range" in cfg:
        lo, hi = len_range or cfg["len_range"]
        b = batch or cfg["batch"]
        lengths = rng.integers(lo, hi + 1, size=b).astype(np.int64)
        if "long_len" in cfg:   # one long context at a seeded position
            lengths[int(rng.integers(b))] = cfg["long_len"]
    else:
        lengths = np.asarray(cfg["lens"], dtype=np.int64)
        if batch is not None:   # the fixed lengths, cycled or cut to the batch
            lengths = np.resize(lengths, batch)
    needed = int(sum(blocks_for(l, bs) for l in lengths))
    pool = cfg["pool"] if pool is None else pool
    if pool == "1.5x":
        n_blocks = int(math.ceil(1.5 * needed))
    elif pool == "exact":
        n_blocks = needed
    else:
        n_blocks = int(pool)
    n_blocks = max(n_blocks, needed, 1)
    perm = rng.permutation(n_blocks).astype(np.int32)
    tables = tables_from_perm(lengths, perm, bs)
    return CaseStructure(name=name, seed=seed, block_size=bs, lengths=lengths,
                         num_blocks=n_blocks, perm=perm, tables=tables,
                         slots=slots_at(lengths, tables, bs))


def make_case(name: str, device="cpu", **overrides) -> DecodeCase:
    """Build the seeded inputs of workload ``name`` on ``device``.

    ``batch``/``lens``/``len_range``/``block_size``/``pool``/``seed`` override
    the workload's values to get the same shape at a size the oracle finishes
    in seconds; ``num_q_heads``/``num_kv_heads``/``head_dim``/``dtype`` give
    other head shapes with the same structure.  The shared-prefix workload is built by ``shared_plan`` and
    ``shared_tensors``.
    """
    shape = {k: overrides.pop(k) for k in ("num_q_heads", "num_kv_heads", "head_dim", "dtype")
             if k in overrides}
    st = case_structure(name, **overrides)
    cfg = {**CONFIGS[name], **shape}
    hq, hkv, d, dt = cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    bs, n_blocks = st.block_size, st.num_blocks
    gen = torch.Generator(device=device).manual_seed(st.seed)
    B = len(st.lengths)
    q = _randn(gen, (B, hq, d), device, dt)
    kc = _pool(gen, n_blocks, hkv, bs * d, device, dt)
    vc = _pool(gen, n_blocks, hkv, bs * d, device, dt)
    nk = _randn(gen, (B, hkv, d), device, dt)
    nv = _randn(gen, (B, hkv, d), device, dt)
    return DecodeCase(
        name=name, seed=st.seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=bs, dtype=dt, num_blocks=n_blocks, scale=1.0 / math.sqrt(d),
        context_lens=st.lengths.astype(np.int32), block_tables=st.tables, perm=st.perm,
        query=q, key_cache=kc, value_cache=vc, new_key=nk, new_value=nv,
        slot_mapping=st.slots, partition_size=int(cfg.get("partition_size", 0)))


@dataclass
class SharedPrefixPlan:
    """Integer plan of the shared-prefix workload (no tensors).

    A parent sequence holds a ``prompt``-token prompt; ``batch - 1`` forks
    share all its blocks; sequence i then appends ``tails[i]`` private tokens.
    Each decode step forks every sequence into a shadow that shares all its
    blocks, appends one token to each of the ``batch`` sequences (ascending
    id), and frees the shadows afterwards.
    """
    seed: int
    batch: int
    prompt: int
    tails: np.ndarray        # int64 [batch]
    block_size: int
    num_blocks: int
    perm: np.ndarray         # int32 [num_blocks]


def shared_plan(*, batch: Optional[int] = None, prompt: Optional[int] = None,
                tail_range=None, seed: Optional[int] = None,
                block_size: Optional[int] = None) -> SharedPrefixPlan:
    cfg = CONFIGS["shared"]
    seed = seed_for("shared") if seed is None else seed
    b = batch or cfg["batch"]
    p = cfg["prompt"] if prompt is None else prompt
    lo, hi = tail_range or cfg["tail_range"]
    bs = block_size or cfg["block_size"]
    rng = np.random.default_rng(seed)
    tails = rng.integers(lo, hi + 1, size=b).astype(np.int64)
    # Blocks alive at the peak of a step: the shared prompt, every private
    # tail, and one new block per sequence (fresh block or CoW destination).
    needed = blocks_for(p, bs) + int(sum(blocks_for(t, bs) + 1 for t in tails))
    n_blocks = int(math.ceil(1.5 * needed))
    perm = rng.permutation(n_blocks).astype(np.int32)
    return SharedPrefixPlan(seed=seed, batch=b, prompt=p, tails=tails,
                            block_size=bs, num_blocks=n_blocks, perm=perm)


def shared_tensors(plan: SharedPrefixPlan, device="cpu"):
    """Float tensors of the shared-prefix workload: q, pools, new key/value."""
    cfg = CONFIGS["shared"]
    hq, hkv, d, dt = cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"], cfg["dtype"]
    gen = torch.Generator(device=device).manual_seed(plan.seed)
    q = _randn(gen, (plan.batch, hq, d), device, dt)
    kc = _pool(gen, plan.num_blocks, hkv, plan.block_size * d, device, dt)
    vc = _pool(gen, plan.num_blocks, hkv, plan.block_size * d, device, dt)
    nk = _randn(gen, (plan.batch, hkv, d), device, dt)
    nv = _randn(gen, (plan.batch, hkv, d), device, dt)
    return dict(query=q, key_cache=kc, value_cache=vc, new_key=nk, new_value=nv,
                num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dt,
                scale=1.0 / math.sqrt(d))


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bits of a bf16 tensor (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_array(t: torch.Tensor) -> np.ndarray:
    """Host copy of a pool/query tensor as the oracle reads it (fp32 or bf16 bits)."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().contiguous().numpy()
