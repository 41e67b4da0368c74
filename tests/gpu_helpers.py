"""Shared pieces of the GPU parity tests: run the HIP path through the
binding, run the oracle on host copies of the very same tensors, compare."""
import numpy as np
import torch

import oracle
import workloads as W

TOL = {"fp32": 1e-5, "bf16": 2e-2}


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda") if dtype is None else t.to(device="cuda", dtype=dtype)


def gpu_decode(pa, case, partition_size=0, out_dtype=None, tables=None, lens=None, query=None,
               key_cache=None, value_cache=None, max_context_len=None, kv_reused=False):
    q = case.query if query is None else query
    out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device="cuda")
    tab = to_dev(case.block_tables if tables is None else tables)
    ln = to_dev(case.context_lens if lens is None else lens)
    mcl = int(ln.max().item()) if max_context_len is None else max_context_len
    pa.paged_attention_decode(
        out, q, case.key_cache if key_cache is None else key_cache,
        case.value_cache if value_cache is None else value_cache, tab, ln,
        num_kv_heads=case.num_kv_heads, block_size=case.block_size, max_context_len=mcl,
        scale=case.scale, partition_size=partition_size, num_blocks=case.num_blocks,
        kv_reused=kv_reused)
    torch.cuda.synchronize()
    return out


def oracle_decode(case, idx=None, threads=16, tables=None, lens=None, query=None, pools=None):
    q = W.host_array(case.query if query is None else query)
    kp, vp = pools if pools is not None else (W.host_array(case.key_cache),
                                             W.host_array(case.value_cache))
    tab = case.block_tables if tables is None else tables
    ln = case.context_lens if lens is None else lens
    if idx is not None:
        q, tab, ln = q[idx], tab[idx], ln[idx]
    return oracle.paged_attention(q, kp, vp, tab, ln, num_kv_heads=case.num_kv_heads,
                                  head_dim=case.head_dim, block_size=case.block_size,
                                  scale=case.scale, num_blocks=case.num_blocks, threads=threads)


def max_abs_err(gpu_out, ref):
    return float(np.max(np.abs(gpu_out.double().cpu().numpy() - ref))) if ref.size else 0.0
