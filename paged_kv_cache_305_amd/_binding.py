"""ctypes binding of libpagedattn.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels or its host
allocator.  PyTorch provides device memory (tensors) and streams; this module
checks tensor placement/dtype/contiguity, derives sizes, and passes
``data_ptr()`` values and the current HIP stream across the C ABI.  If the
library is missing it is built once from source; if it cannot be loaded,
every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_OUT_OF_BLOCKS = -3
PA_ERR_UNKNOWN_SEQ = -4
PA_ERR_HIP = -5
PA_FP32 = 0
PA_BF16 = 1
PA_PARTITION_BALANCED = -1
PA_PARTITION_AUTO = -2
PA_AUTO_WHOLE_MAX_LEN = 256
PA_DECODE_KV_REUSED = 1

# Every symbol include/pagedattn.h declares.
EXPORTS = (
    "pa_last_error", "pa_version",
    "pa_paged_attention_decode", "pa_paged_attention_decode_append",
    "pa_paged_attention_decode_noalloc",
    "pa_paged_attention_decode_prefix", "pa_paged_attention_prefix_workspace_bytes",
    "pa_paged_attention_workspace_bytes", "pa_resolve_partition", "pa_set_timing_events",
    "pa_set_balance_weights",
    "pa_reshape_and_cache", "pa_copy_blocks", "pa_swap_blocks",
    "pa_reshape_and_cache_layers", "pa_copy_blocks_layers",
    "pa_allocator_create", "pa_allocator_destroy", "pa_allocator_num_free",
    "pa_allocator_block_size", "pa_seq_create", "pa_seq_fork", "pa_seq_append_slot",
    "pa_seq_free", "pa_seq_block_table", "pa_seq_len", "pa_block_refcount",
    "pa_build_block_tables", "pa_allocator_set_swap_space", "pa_allocator_num_free_host",
    "pa_host_block_refcount", "pa_seq_is_swapped", "pa_seqs_swap_out", "pa_seqs_swap_in",
)


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("status %d: %s" % (status, message))
        self.status = status


_lib = None


def _declare(lib):
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    p_i32, p_i64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    sig = {
        "pa_last_error": (ctypes.c_char_p, []),
        "pa_version": (i32, []),
        "pa_paged_attention_decode": (i32, [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            i64, i32, f32, i32, i32, i32, ctypes.c_uint32, vp, sz,
                                            vp]),
        "pa_paged_attention_decode_append": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                                   i32, i32, i32, i32, i64, i32, f32, i32, i32,
                                                   i32, ctypes.c_uint32, vp, sz, vp]),
        "pa_paged_attention_decode_noalloc": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                                    i32, i32, i32, i32, i64, i32, f32, i32, i32,
                                                    i32, ctypes.c_uint32, vp]),
        "pa_paged_attention_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32, i32]),
        "pa_resolve_partition": (i32, [i32, i32]),
        "pa_paged_attention_decode_prefix": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                                   i32, i32, i32, i32, i64, i32, f32, i32, i32,
                                                   i32, ctypes.c_uint32, vp, sz, vp]),
        "pa_paged_attention_prefix_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32, i32]),
        "pa_set_timing_events": (i32, [vp, vp, vp, vp]),
        "pa_set_balance_weights": (i32, [vp, i32]),
        "pa_reshape_and_cache": (i32, [vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32, vp]),
        "pa_copy_blocks": (i32, [vp, vp, vp, i32, i32, i32, i32, i64, i32, vp]),
        "pa_swap_blocks": (i32, [vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i64, i32, vp]),
        "pa_reshape_and_cache_layers": (i32, [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i64,
                                              i32, vp]),
        "pa_copy_blocks_layers": (i32, [vp, vp, i32, vp, i32, i32, i32, i32, i64, i32, vp]),
        "pa_allocator_set_swap_space": (i32, [vp, i64]),
        "pa_allocator_num_free_host": (i64, [vp]),
        "pa_host_block_refcount": (i32, [vp, i32]),
        "pa_seq_is_swapped": (i32, [vp, i64]),
        "pa_seqs_swap_out": (i32, [vp, vp, i32, vp, i32, p_i32]),
        "pa_seqs_swap_in": (i32, [vp, vp, i32, vp, i32, p_i32]),
        "pa_allocator_create": (vp, [i64, i32, vp]),
        "pa_allocator_destroy": (None, [vp]),
        "pa_allocator_num_free": (i64, [vp]),
        "pa_allocator_block_size": (i32, [vp]),
        "pa_seq_create": (i32, [vp, i64, i64]),
        "pa_seq_fork": (i32, [vp, i64, i64]),
        "pa_seq_append_slot": (i32, [vp, i64, p_i64, p_i64, p_i64]),
        "pa_seq_free": (i32, [vp, i64]),
        "pa_seq_block_table": (i32, [vp, i64, vp, i32, p_i32]),
        "pa_seq_len": (i64, [vp, i64]),
        "pa_block_refcount": (i32, [vp, i32]),
        "pa_build_block_tables": (i32, [vp, vp, i32, i32, i32, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load():
    """Load (building once if absent) libpagedattn.so; returns the ctypes handle."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: its HIP runtime is then the one the library binds to
    # (both carry the same SONAME), so torch's stream handles are valid here.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    _declare(lib)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError("two HIP runtimes are mapped (%s); load torch before this library"
                           % ", ".join(sorted(runtimes)))
    _lib = lib
    return lib


def _err(status: int) -> PagedAttnError:
    msg = load().pa_last_error()
    return PagedAttnError(status, msg.decode() if msg else "")


def _check(status: int):
    if status != PA_OK:
        raise _err(status)


# ---- tensors -----------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code_of(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return PA_FP32
    if dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % dtype)


def _dtype_code(t) -> int:
    return _dtype_code_of(t.dtype)


def _dev(t, name, device=None):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    return t


def _stream(device, stream) -> int:
    if stream is not None:
        return int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    return int(_torch().cuda.current_stream(device).cuda_stream)


def key_cache_shape(num_blocks, num_kv_heads, head_dim, block_size, dtype):
    """[num_blocks, Hkv, d / x, block_size, x], x = 16 bytes / element size."""
    x = 16 // _torch().empty((), dtype=dtype).element_size()
    return (num_blocks, num_kv_heads, head_dim // x, block_size, x)


def value_cache_shape(num_blocks, num_kv_heads, head_dim, block_size):
    """[num_blocks, Hkv, block_size / 16, d, 16]: each feature's tokens in
    groups of 16, one group per 16-token tile (block_size a multiple of 16)."""
    if block_size % 16:
        raise ValueError("block_size must be a multiple of 16, got %d" % block_size)
    return (num_blocks, num_kv_heads, block_size // 16, head_dim, 16)


def allocate_pools(num_blocks, num_kv_heads, head_dim, block_size, dtype, device="cuda"):
    """Empty key and value pools in the library's layout."""
    torch = _torch()
    k = torch.empty(key_cache_shape(num_blocks, num_kv_heads, head_dim, block_size, dtype),
                    dtype=dtype, device=device)
    v = torch.empty(value_cache_shape(num_blocks, num_kv_heads, head_dim, block_size),
                    dtype=dtype, device=device)
    return k, v


def set_timing_events(main_start=None, main_end=None, merge_start=None, merge_end=None):
    """Stamp these torch.cuda.Events with the start and end of the main attention
    kernel (and of the merge kernel) of every later decode call from this thread;
    all None stops.  The runtime stamps them from the kernels themselves, so
    main_start.elapsed_time(main_end) is the kernel's duration."""
    def h(e):
        if e is None:
            return None
        if not int(e.cuda_event):
            raise ValueError("record the event once first: torch creates HIP events lazily")
        return int(e.cuda_event)
    _check(load().pa_set_timing_events(h(main_start), h(main_end), h(merge_start),
                                       h(merge_end)))


def set_balance_weights(weights=None):
    """Per-XCD tile shares of the balanced split (8 ints in [1, 1000]); None restores
    the default (even-numbered XCDs 115, odd 100)."""
    if weights is None:
        _check(load().pa_set_balance_weights(None, 0))
        return
    w = np.ascontiguousarray(np.asarray(weights, dtype=np.int32))
    _check(load().pa_set_balance_weights(w.ctypes.data, int(w.size)))


def resolve_partition(partition_size: int, max_context_len: int) -> int:
    """The split a decode call with these arguments runs (PA_PARTITION_AUTO
    gives 0 or PA_PARTITION_BALANCED; other values are returned as they are)."""
    return int(load().pa_resolve_partition(int(partition_size), int(max_context_len)))


def paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                    max_context_len, partition_size, kv_dtype) -> int:
    """kv_dtype: PA_FP32 / PA_BF16 or a torch dtype."""
    code = kv_dtype if isinstance(kv_dtype, int) else \
        {_torch().float32: PA_FP32, _torch().bfloat16: PA_BF16}[kv_dtype]
    return int(load().pa_paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                         head_dim, max_context_len,
                                                         partition_size, code))


def paged_attention_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           max_context_len, prefix_len, kv_dtype) -> int:
    lib = load()
    return int(lib.pa_paged_attention_prefix_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, prefix_len,
        _dtype_code_of(kv_dtype)))


def _new_token_ptrs(new_key, new_value, slot_mapping, B, num_kv_heads, d, dtype, dev,
                    cow_src=None):
    """Device pointers of a step's new tokens (all three given) and of the
    optional in-launch copy-on-write sources, or zeros (none)."""
    if new_key is None and new_value is None and slot_mapping is None:
        if cow_src is not None:
            raise ValueError("cow_src needs the new tokens")
        return 0, 0, 0, 0
    if new_key is None or new_value is None or slot_mapping is None:
        raise ValueError("new_key, new_value and slot_mapping go together")
    for t, n in ((new_key, "new_key"), (new_value, "new_value"), (slot_mapping, "slot_mapping")):
        _dev(t, n, dev)
    if tuple(new_key.shape) != (B, num_kv_heads, d) or new_value.shape != new_key.shape:
        raise ValueError("new_key and new_value must be [num_seqs, num_kv_heads, head_dim]")
    if new_key.dtype != dtype or new_value.dtype != dtype:
        raise TypeError("new_key and new_value must have the pools' dtype")
    if slot_mapping.dtype != _torch().int64 or slot_mapping.shape != (B,):
        raise ValueError("slot_mapping must be int64 [num_seqs]")
    cow = 0
    if cow_src is not None:
        _dev(cow_src, "cow_src", dev)
        if cow_src.dtype != _torch().int64 or cow_src.shape != (B,):
            raise ValueError("cow_src must be int64 [num_seqs]")
        cow = cow_src.data_ptr()
    return new_key.data_ptr(), new_value.data_ptr(), slot_mapping.data_ptr(), cow


def paged_attention_decode_prefix(out, query, key_cache, value_cache, block_tables,
                                  context_lens, *, prefix_len: int, num_kv_heads: int,
                                  block_size: int, max_context_len: int, scale: float,
                                  workspace=None, num_blocks: Optional[int] = None,
                                  new_key=None, new_value=None, slot_mapping=None,
                                  cow_src=None, stream=None):
    """Decode attention when every sequence's first prefix_len tokens are the
    same physical blocks (sequence 0's): those are read once for all rows.
    new_key, new_value, slot_mapping and cow_src as in paged_attention_decode
    (each new token after the prefix)."""
    lib = load()
    dev = query.device
    for t, n in ((out, "out"), (query, "query"), (key_cache, "key_cache"),
                 (value_cache, "value_cache"), (block_tables, "block_tables"),
                 (context_lens, "context_lens")):
        _dev(t, n, dev)
    torch = _torch()
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    B, hq, d = query.shape
    if tuple(out.shape) != (B, hq, d):
        raise ValueError("out must have the query's shape")
    nb = int(key_cache.shape[0]) if num_blocks is None else int(num_blocks)
    news = _new_token_ptrs(new_key, new_value, slot_mapping, B, num_kv_heads, d, query.dtype, dev,
                           cow_src)
    need = paged_attention_prefix_workspace_bytes(B, hq, num_kv_heads, d, max_context_len,
                                                  prefix_len, query.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.pa_paged_attention_decode_prefix(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), *news,
        block_tables.data_ptr(), context_lens.data_ptr(), B, hq, num_kv_heads, d, block_size,
        int(block_tables.shape[1]), nb, int(max_context_len), float(scale), int(prefix_len),
        _dtype_code(query), _dtype_code(out), 0, _dev(workspace, "workspace", dev).data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(dev, stream)))
    return out


def _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, num_kv_heads,
                 block_size, max_context_len, scale, partition_size, num_blocks, kv_reused,
                 new_key, new_value, slot_mapping, cow_src):
    """Checked pointers and sizes of a decode call: (appending, new-token
    pointers, arguments after them up to the flags)."""
    dev = query.device
    appending = new_key is not None or new_value is not None or slot_mapping is not None
    if cow_src is not None and not appending:
        raise ValueError("cow_src needs the new tokens")
    for t, n in ((out, "out"), (query, "query"), (key_cache, "key_cache"),
                 (value_cache, "value_cache"), (block_tables, "block_tables"),
                 (context_lens, "context_lens")):
        _dev(t, n, dev)
    torch = _torch()
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if query.dim() != 3:
        raise ValueError("query must be [num_seqs, num_q_heads, head_dim]")
    B, hq, d = query.shape
    if tuple(out.shape) != (B, hq, d):
        raise ValueError("out must have the query's shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    if key_cache.dtype != query.dtype or value_cache.dtype != query.dtype:
        raise TypeError("query and pools must share a dtype")
    nb = int(key_cache.shape[0]) if num_blocks is None else int(num_blocks)
    chunk = num_kv_heads * d * block_size
    if key_cache.numel() < nb * chunk or value_cache.numel() < nb * chunk:
        raise ValueError("pools hold fewer than num_blocks blocks")
    news = _new_token_ptrs(new_key, new_value, slot_mapping, B, num_kv_heads, d, query.dtype, dev,
                           cow_src)
    tail = (block_tables.data_ptr(), context_lens.data_ptr(), B, hq, num_kv_heads, d, block_size,
            int(block_tables.shape[1]), nb, int(max_context_len), float(scale),
            int(partition_size), _dtype_code(query), _dtype_code(out),
            PA_DECODE_KV_REUSED if kv_reused else 0)
    return appending, news, tail


def paged_attention_decode(out, query, key_cache, value_cache, block_tables, context_lens, *,
                           num_kv_heads: int, block_size: int, max_context_len: int,
                           scale: float, partition_size: int = 0, workspace=None,
                           num_blocks: Optional[int] = None, kv_reused: bool = False,
                           new_key=None, new_value=None, slot_mapping=None, cow_src=None,
                           stream=None):
    """out[B, Hq, d] = softmax(scale q K^T) V per sequence, K/V read through the tables.

    kv_reused: some physical blocks are read by several sequences (shared
    prefixes): keep K/V in the caches instead of streaming them.

    new_key, new_value ([B, Hkv, d]) and slot_mapping (int64 [B]), given
    together: each sequence's last position is this new token, written into
    its slot by the same launch (pa_paged_attention_decode_append).
    cow_src (int64 [B], optional with them): the copy-on-write source of
    each sequence's new-token block, copied inside the launch (-1: none)."""
    lib = load()
    dev = query.device
    appending, news, tail = _decode_args(out, query, key_cache, value_cache, block_tables,
                                         context_lens, num_kv_heads, block_size, max_context_len,
                                         scale, partition_size, num_blocks, kv_reused, new_key,
                                         new_value, slot_mapping, cow_src)
    B, hq, d = query.shape
    need = paged_attention_workspace_bytes(B, hq, num_kv_heads, d, max_context_len,
                                           partition_size, query.dtype)
    if need and workspace is None:
        workspace = _torch().empty(need, dtype=_torch().uint8, device=dev)
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (
        _dev(workspace, "workspace", dev).data_ptr(), workspace.numel() * workspace.element_size())
    tail = tail + (ws_ptr, ws_bytes, _stream(dev, stream))
    if appending:
        _check(lib.pa_paged_attention_decode_append(
            out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            *news, *tail))
    else:
        _check(lib.pa_paged_attention_decode(
            out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            *tail))
    return out


def paged_attention_decode_noalloc(out, query, key_cache, value_cache, block_tables,
                                   context_lens, *, num_kv_heads: int, block_size: int,
                                   max_context_len: int, scale: float, partition_size: int = 0,
                                   num_blocks: Optional[int] = None, kv_reused: bool = False,
                                   new_key=None, new_value=None, slot_mapping=None, cow_src=None,
                                   stream=None):
    """paged_attention_decode without a workspace: the library's own device
    array holds the call's scratch, so nothing is allocated (callers that
    cannot allocate, e.g. under graph capture).  Calls that would need more
    scratch than the array holds raise PagedAttnError; calls that overlap on
    one GPU race."""
    lib = load()
    _, news, tail = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                                 num_kv_heads, block_size, max_context_len, scale, partition_size,
                                 num_blocks, kv_reused, new_key, new_value, slot_mapping, cow_src)
    _check(lib.pa_paged_attention_decode_noalloc(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), *news,
        *tail, _stream(query.device, stream)))
    return out


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, *, block_size: int,
                      num_blocks: Optional[int] = None, stream=None):
    """Write key/value [T, Hkv, d] into their slots of the pools (bit copy)."""
    lib = load()
    dev = key.device
    for t, n in ((key, "key"), (value, "value"), (key_cache, "key_cache"),
                 (value_cache, "value_cache"), (slot_mapping, "slot_mapping")):
        _dev(t, n, dev)
    if slot_mapping.dtype != _torch().int64:
        raise TypeError("slot_mapping must be int64")
    if key.dim() != 3 or key.shape != value.shape:
        raise ValueError("key and value must be [num_tokens, num_kv_heads, head_dim]")
    if not (key.dtype == value.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("key, value and pools must share a dtype")
    T, hkv, d = key.shape
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    nb = int(key_cache.shape[0]) if num_blocks is None else int(num_blocks)
    _check(lib.pa_reshape_and_cache(
        key.data_ptr(), value.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        slot_mapping.data_ptr(), T, hkv, d, block_size, nb, _dtype_code(key),
        _stream(dev, stream)))


def copy_blocks(key_cache, value_cache, block_mapping, *, num_kv_heads: int, head_dim: int,
                block_size: int, num_blocks: Optional[int] = None, stream=None):
    """Copy whole blocks src -> dst in both pools; block_mapping is int64 [n, 2]."""
    lib = load()
    dev = key_cache.device
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache"),
                 (block_mapping, "block_mapping")):
        _dev(t, n, dev)
    if block_mapping.dtype != _torch().int64:
        raise TypeError("block_mapping must be int64")
    if block_mapping.numel() % 2:
        raise ValueError("block_mapping must be [num_pairs, 2]")
    nb = int(key_cache.shape[0]) if num_blocks is None else int(num_blocks)
    _check(lib.pa_copy_blocks(
        key_cache.data_ptr(), value_cache.data_ptr(), block_mapping.data_ptr(),
        block_mapping.numel() // 2, num_kv_heads, head_dim, block_size, nb,
        _dtype_code(key_cache), _stream(dev, stream)))


def swap_blocks(dst_key_cache, dst_value_cache, src_key_cache, src_value_cache, block_mapping,
                *, num_kv_heads: int, head_dim: int, block_size: int, stream=None):
    """Copy whole blocks (src block, dst block) = block_mapping[k] from the src
    pools to the dst pools.  Each pool, and block_mapping (int64 [n, 2]), is
    either on the GPU or in pinned host memory (pin_memory=True)."""
    lib = load()
    torch = _torch()
    tensors = ((dst_key_cache, "dst_key_cache"), (dst_value_cache, "dst_value_cache"),
               (src_key_cache, "src_key_cache"), (src_value_cache, "src_value_cache"),
               (block_mapping, "block_mapping"))
    devs = {t.device for t, _ in tensors if t.is_cuda}
    if len(devs) != 1:
        raise ValueError("swap_blocks needs tensors on exactly one GPU (the others pinned)")
    dev = devs.pop()
    for t, n in tensors:
        if not t.is_cuda and not t.is_pinned():
            raise ValueError("%s must be on the GPU or in pinned host memory" % n)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    if block_mapping.dtype != torch.int64 or block_mapping.numel() % 2:
        raise ValueError("block_mapping must be int64 [num_pairs, 2]")
    if dst_key_cache.dtype != src_key_cache.dtype:
        raise TypeError("pools must share a dtype")
    _check(lib.pa_swap_blocks(
        dst_key_cache.data_ptr(), dst_value_cache.data_ptr(), src_key_cache.data_ptr(),
        src_value_cache.data_ptr(), block_mapping.data_ptr(), block_mapping.numel() // 2,
        num_kv_heads, head_dim, block_size, int(src_key_cache.shape[0]),
        int(dst_key_cache.shape[0]), _dtype_code(src_key_cache), _stream(dev, stream)))


def pointer_array(tensors, device):
    """int64 device tensor of the tensors' data pointers (for the per-layer calls).
    Build it once per set of pools: it is an upload."""
    torch = _torch()
    device = torch.device(device)
    if device.type == "cuda" and device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    for t in tensors:
        _dev(t, "per-layer tensor", device)
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=device)


def reshape_and_cache_layers(key_ptrs, value_ptrs, key_cache_ptrs, value_cache_ptrs,
                             slot_mapping, *, num_layers: int, num_kv_heads: int, head_dim: int,
                             block_size: int, num_blocks: int, dtype, stream=None):
    """reshape_and_cache on every layer in one launch; the *_ptrs are
    pointer_array() tensors of the per-layer keys, values and pools."""
    lib = load()
    dev = slot_mapping.device
    for t, n in ((key_ptrs, "key_ptrs"), (value_ptrs, "value_ptrs"),
                 (key_cache_ptrs, "key_cache_ptrs"), (value_cache_ptrs, "value_cache_ptrs")):
        _dev(t, n, dev)
        if t.dtype != _torch().int64 or t.numel() != num_layers:
            raise ValueError("%s must be int64 [num_layers]" % n)
    _check(lib.pa_reshape_and_cache_layers(
        key_ptrs.data_ptr(), value_ptrs.data_ptr(), key_cache_ptrs.data_ptr(),
        value_cache_ptrs.data_ptr(), int(num_layers), slot_mapping.data_ptr(),
        int(slot_mapping.numel()), num_kv_heads, head_dim, block_size, int(num_blocks),
        _dtype_code_of(dtype), _stream(dev, stream)))


def copy_blocks_layers(key_cache_ptrs, value_cache_ptrs, block_mapping, *, num_layers: int,
                       num_kv_heads: int, head_dim: int, block_size: int, num_blocks: int, dtype,
                       stream=None):
    """copy_blocks on every layer in one launch (pointer_array() pools)."""
    lib = load()
    dev = block_mapping.device
    for t, n in ((key_cache_ptrs, "key_cache_ptrs"), (value_cache_ptrs, "value_cache_ptrs")):
        _dev(t, n, dev)
        if t.dtype != _torch().int64 or t.numel() != num_layers:
            raise ValueError("%s must be int64 [num_layers]" % n)
    if block_mapping.dtype != _torch().int64 or block_mapping.numel() % 2:
        raise ValueError("block_mapping must be int64 [num_pairs, 2]")
    _check(lib.pa_copy_blocks_layers(
        key_cache_ptrs.data_ptr(), value_cache_ptrs.data_ptr(), int(num_layers),
        block_mapping.data_ptr(), block_mapping.numel() // 2, num_kv_heads, head_dim,
        block_size, int(num_blocks), _dtype_code_of(dtype), _stream(dev, stream)))


# ---- allocator -----------------------------------------------------------------

class BlockAllocator:
    """Host block allocator (free list, refcounts, copy-on-write) owned by the library."""

    def __init__(self, num_blocks: int, block_size: int,
                 initial_free_order: Optional[Sequence[int]] = None):
        lib = load()
        self._lib = lib
        order = None
        ptr = None
        if initial_free_order is not None:
            order = np.ascontiguousarray(np.asarray(initial_free_order, dtype=np.int32))
            if order.shape != (num_blocks,):
                raise ValueError("initial_free_order must hold num_blocks entries")
            ptr = order.ctypes.data
        h = lib.pa_allocator_create(int(num_blocks), int(block_size), ptr)
        if not h:
            raise _err(PA_ERR_INVALID_ARG)
        self._h = ctypes.c_void_p(h)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def num_free(self) -> int:
        return int(self._lib.pa_allocator_num_free(self._h))

    def create(self, seq_id: int, num_tokens: int):
        _check(self._lib.pa_seq_create(self._h, int(seq_id), int(num_tokens)))

    def fork(self, parent_id: int, child_id: int):
        _check(self._lib.pa_seq_fork(self._h, int(parent_id), int(child_id)))

    def append_slot(self, seq_id: int):
        """Returns (slot, cow_src, cow_dst); the pair is (-1, -1) when nothing is copied."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(self._lib.pa_seq_append_slot(self._h, int(seq_id), ctypes.byref(slot),
                                            ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, src.value, dst.value

    def free(self, seq_id: int):
        _check(self._lib.pa_seq_free(self._h, int(seq_id)))

    def seq_len(self, seq_id: int) -> int:
        return int(self._lib.pa_seq_len(self._h, int(seq_id)))

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_block_refcount(self._h, int(block)))

    def block_table(self, seq_id: int) -> list:
        n = ctypes.c_int32()
        L = self.seq_len(seq_id)
        cap = max(1, -(-max(L, 0) // self.block_size))
        buf = np.zeros(cap, dtype=np.int32)
        _check(self._lib.pa_seq_block_table(self._h, int(seq_id), buf.ctypes.data, cap,
                                            ctypes.byref(n)))
        return buf[:n.value].tolist()

    def set_swap_space(self, num_host_blocks: int):
        _check(self._lib.pa_allocator_set_swap_space(self._h, int(num_host_blocks)))

    def num_free_host(self) -> int:
        return int(self._lib.pa_allocator_num_free_host(self._h))

    def host_refcount(self, block: int) -> int:
        return int(self._lib.pa_host_block_refcount(self._h, int(block)))

    def is_swapped(self, seq_id: int) -> bool:
        r = int(self._lib.pa_seq_is_swapped(self._h, int(seq_id)))
        if r < 0:
            raise _err(PA_ERR_UNKNOWN_SEQ)
        return bool(r)

    def _swap(self, fn, seq_ids):
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        cap = 0
        for i in ids.tolist():
            cap += -(-max(self.seq_len(i), 0) // self.block_size)
        pairs = np.empty((max(cap, 1), 2), dtype=np.int64)
        n = ctypes.c_int32()
        _check(fn(self._h, ids.ctypes.data, int(ids.shape[0]), pairs.ctypes.data, cap,
                  ctypes.byref(n)))
        return pairs[:n.value].copy()

    def swap_out(self, seq_ids):
        """Preempt these sequences to the swap space; returns int64 [n, 2]
        (device block, swap block) pairs to copy with swap_blocks."""
        return self._swap(self._lib.pa_seqs_swap_out, seq_ids)

    def swap_in(self, seq_ids):
        """Bring swapped sequences back; returns (swap block, device block) pairs."""
        return self._swap(self._lib.pa_seqs_swap_in, seq_ids)

    def build_block_tables(self, seq_ids, max_blocks: int, pad: int = 0):
        """Host int32 tables [n, max_blocks] (padded) and lengths [n] for upload."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = int(ids.shape[0])
        tabs = np.empty((n, max_blocks), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        _check(self._lib.pa_build_block_tables(self._h, ids.ctypes.data, n, int(max_blocks),
                                               int(pad), tabs.ctypes.data, lens.ctypes.data))
        return tabs, lens
