"""CPU oracle for the paged decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
binding) never imports, links or runs anything here, and this package never
imports the product.

Contents:
  * ``oracle.c`` -- plain C, fp64: gather-then-naive-softmax attention,
    the reshape_and_cache scatter, the copy_blocks copy and the swap_blocks
    copy between pools (see its header for the passages each follows and
    the pool layout it addresses).
  * ``alloc_model`` -- a plain Python model of the block allocator.

Every function here is pinned by ``tests/test_oracle_*.py`` against
brute-force unpaged attention, closed forms, invariances and the pages'
worked example.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

FP32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-Werror", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.oracle_paged_attention.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                               i32, i64, ctypes.c_double, i32, i32]
        lib.oracle_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32]
        lib.oracle_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i64, i32]
        lib.oracle_swap_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i64, i32]
        for f in (lib.oracle_paged_attention, lib.oracle_reshape_and_cache,
                  lib.oracle_copy_blocks, lib.oracle_swap_blocks):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return FP32
    if a.dtype in (np.uint16, np.int16):
        return BF16
    raise TypeError("oracle takes fp32 arrays or bf16 bits as uint16, got %s" % a.dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


def paged_attention(query, key_cache, value_cache, block_tables, context_lens, *,
                    num_kv_heads: int, head_dim: int, block_size: int, scale: float,
                    num_blocks: int, threads: int = 1) -> np.ndarray:
    """fp64 [B, Hq, d] output of plain softmax attention read through the tables."""
    q = _c(query)
    kc, vc = _c(key_cache), _c(value_cache)
    dt = _dtype_code(q)
    if _dtype_code(kc) != dt or _dtype_code(vc) != dt:
        raise TypeError("query and pools must share a dtype")
    tab = _c(block_tables, np.int32)
    lens = _c(context_lens, np.int32)
    B = int(lens.shape[0])
    hq = int(q.size // max(1, B * head_dim)) if B else 1
    out = np.zeros((B, hq, head_dim), dtype=np.float64)
    rc = _load().oracle_paged_attention(
        _ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(tab), _ptr(lens), B, hq, num_kv_heads,
        head_dim, block_size, int(tab.shape[1]) if tab.ndim == 2 else 1, int(num_blocks),
        float(scale), dt, int(threads))
    if rc != 0:
        raise ValueError("oracle_paged_attention failed (%d)" % rc)
    return out


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, *, num_kv_heads: int,
                      head_dim: int, block_size: int, num_blocks: int) -> None:
    """In-place scatter of each token's K/V into its slot (host arrays)."""
    k, v = _c(key), _c(value)
    for a in (key_cache, value_cache):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("pools must be contiguous (written in place)")
    s = _c(slot_mapping, np.int64)
    rc = _load().oracle_reshape_and_cache(
        _ptr(k), _ptr(v), _ptr(key_cache), _ptr(value_cache), _ptr(s), int(s.shape[0]),
        num_kv_heads, head_dim, block_size, int(num_blocks), _dtype_code(key_cache))
    if rc != 0:
        raise ValueError("oracle_reshape_and_cache failed (%d)" % rc)


def copy_blocks(key_cache, value_cache, block_mapping, *, num_kv_heads: int, head_dim: int,
                block_size: int, num_blocks: int) -> None:
    """In-place whole-block copies src -> dst, all sources read first."""
    for a in (key_cache, value_cache):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("pools must be contiguous (written in place)")
    m = _c(block_mapping, np.int64).reshape(-1, 2)
    rc = _load().oracle_copy_blocks(
        _ptr(key_cache), _ptr(value_cache), _ptr(m), int(m.shape[0]), num_kv_heads, head_dim,
        block_size, int(num_blocks), _dtype_code(key_cache))
    if rc != 0:
        raise ValueError("oracle_copy_blocks failed (%d)" % rc)


def swap_blocks(dst_key, dst_value, src_key, src_value, block_mapping, *, num_kv_heads: int,
                head_dim: int, block_size: int) -> None:
    """Whole-block copies from the src pools into the (distinct) dst pools:
    block t of dst becomes block s of src for each pair (s, t)."""
    for a in (dst_key, dst_value):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("destination pools must be contiguous (written in place)")
    m = _c(block_mapping, np.int64).reshape(-1, 2)
    sk, sv = _c(src_key, src_key.dtype), _c(src_value, src_value.dtype)
    rc = _load().oracle_swap_blocks(
        _ptr(dst_key), _ptr(dst_value), _ptr(sk), _ptr(sv), _ptr(m), int(m.shape[0]),
        num_kv_heads, head_dim, block_size, int(sk.shape[0]), int(dst_key.shape[0]),
        _dtype_code(dst_key))
    if rc != 0:
        raise ValueError("oracle_swap_blocks failed (%d)" % rc)
