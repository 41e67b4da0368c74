"""Test-side construction of paged pools from contiguous per-sequence K/V.

Written with numpy reshapes/transposes of whole blocks, independently of the
oracle's per-element index formulas, from the library's stated layout:

    x = 16 / element size
    T = 16 when block_size is a multiple of 16, else T = block_size
    key pool   [num_blocks][Hkv][d / x][block_size][x]
    value pool [num_blocks][Hkv][block_size / T][d][T]

so a mistake in either the oracle's gather or this scatter shows up as a
disagreement with brute-force attention on the contiguous inputs.
"""
from __future__ import annotations

import numpy as np


def x_of(dtype) -> int:
    return 16 // np.dtype(dtype).itemsize


def value_group(block_size: int) -> int:
    return 16 if block_size % 16 == 0 else block_size


def blocks_of(seq_kv: np.ndarray, block_size: int, fill) -> np.ndarray:
    """[L, Hkv, d] -> [nb, Bs, Hkv, d], the tail padded with ``fill``."""
    L, hkv, d = seq_kv.shape
    nb = -(-L // block_size)
    out = np.full((nb * block_size, hkv, d), fill, dtype=seq_kv.dtype)
    out[:L] = seq_kv
    return out.reshape(nb, block_size, hkv, d)


def key_blocks(seq_k: np.ndarray, block_size: int, fill=0) -> np.ndarray:
    """Per-block key chunks in pool layout: [nb, Hkv, d/x, Bs, x]."""
    b = blocks_of(seq_k, block_size, fill)
    nb, bs, hkv, d = b.shape
    x = x_of(seq_k.dtype)
    return b.reshape(nb, bs, hkv, d // x, x).transpose(0, 2, 3, 1, 4)


def value_blocks(seq_v: np.ndarray, block_size: int, fill=0) -> np.ndarray:
    """Per-block value chunks in pool layout: [nb, Hkv, Bs/T, d, T]."""
    b = blocks_of(seq_v, block_size, fill)
    nb, bs, hkv, d = b.shape
    t = value_group(bs)
    return b.reshape(nb, bs // t, t, hkv, d).transpose(0, 3, 1, 4, 2)


def empty_pools(num_blocks, hkv, d, block_size, dtype, fill=0):
    x = x_of(dtype)
    t = value_group(block_size)
    kp = np.full((num_blocks, hkv, d // x, block_size, x), fill, dtype=dtype)
    vp = np.full((num_blocks, hkv, block_size // t, d, t), fill, dtype=dtype)
    return kp, vp


def scatter_sequences(kp, vp, tables, seq_ks, seq_vs, block_size, fill=0):
    """Write each sequence's contiguous K/V into its table's physical blocks."""
    for i, (k, v) in enumerate(zip(seq_ks, seq_vs)):
        if k.shape[0] == 0:
            continue
        kb = key_blocks(k, block_size, fill)
        vb = value_blocks(v, block_size, fill)
        phys = np.asarray(tables[i][:kb.shape[0]])
        kp[phys] = kb.reshape((len(phys),) + kp.shape[1:])
        vp[phys] = vb.reshape((len(phys),) + vp.shape[1:])
    return kp, vp


def gather_sequence(kp, vp, table, L, block_size):
    """Read a sequence back out as contiguous [L, Hkv, d] K and V (test-side)."""
    nb = -(-L // block_size)
    phys = np.asarray(table[:nb])
    kb = kp[phys]                      # [nb, Hkv, d/x, Bs, x]
    nb_, hkv, dx, bs, x = kb.shape
    k = kb.transpose(0, 3, 1, 2, 4).reshape(nb * bs, hkv, dx * x)[:L]
    t = value_group(bs)
    vb = vp[phys].reshape(nb, hkv, bs // t, dx * x, t)   # [nb, Hkv, Bs/T, d, T]
    v = vb.transpose(0, 2, 4, 1, 3).reshape(nb * bs, hkv, dx * x)[:L]
    return k, v
