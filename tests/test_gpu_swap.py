"""swap_blocks and the allocator's swap space on the GPU: preempting
sequences to pinned host memory and bringing them back (inferensys glossary
"Paged Attention", third and fifth paragraphs; crackai.dev "How It Works",
preemption and swapping).  Block copies must equal the oracle's byte for
byte, and swapped-in sequences must attend exactly as before they left."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _random_bf16(shape, gen, pinned):
    """Arbitrary bf16 bit patterns (NaN and Inf included): for bit copies only."""
    t = torch.randint(-32768, 32767, shape, dtype=torch.int16, generator=gen).view(torch.bfloat16)
    return t.pin_memory() if pinned else t.cuda()


def test_block_copies_between_gpu_and_pinned_host_pools_are_bit_exact(gpu):
    gen = torch.Generator().manual_seed(40)
    N, H, hkv, d, bs = 40, 12, 8, 128, 16
    shape = lambda n: (n, hkv, d * bs)
    kc, vc = _random_bf16(shape(N), gen, False), _random_bf16(shape(N), gen, False)
    hk, hv = _random_bf16(shape(H), gen, True), _random_bf16(shape(H), gen, True)
    kw = dict(num_kv_heads=hkv, head_dim=d, block_size=bs)
    # GPU -> host, mapping on the GPU.
    out = np.array([[3, 0], [N - 1, 5], [0, 11], [17, 2]], np.int64)
    ref_k, ref_v = W.host_array(hk).copy(), W.host_array(hv).copy()
    oracle.swap_blocks(ref_k, ref_v, W.host_array(kc), W.host_array(vc), out, **kw)
    gpu.swap_blocks(hk, hv, kc, vc, to_dev(out), **kw)
    torch.cuda.synchronize()
    assert W.host_array(hk).tobytes() == ref_k.tobytes()
    assert W.host_array(hv).tobytes() == ref_v.tobytes()
    # Host -> GPU, mapping in pinned host memory.
    back = np.array([[0, 20], [5, 21], [11, 3], [2, N - 2]], np.int64)
    ref_k, ref_v = W.host_array(kc).copy(), W.host_array(vc).copy()
    oracle.swap_blocks(ref_k, ref_v, W.host_array(hk), W.host_array(hv), back, **kw)
    gpu.swap_blocks(kc, vc, hk, hv, torch.from_numpy(back).pin_memory(), **kw)
    torch.cuda.synchronize()
    assert W.host_array(kc).tobytes() == ref_k.tobytes()
    assert W.host_array(vc).tobytes() == ref_v.tobytes()


def _decode(gpu, q, kc, vc, tabs, lens, hkv, bs):
    out = torch.empty_like(q)
    gpu.paged_attention_decode(out, q, kc, vc, to_dev(tabs), to_dev(lens), num_kv_heads=hkv,
                               block_size=bs, max_context_len=int(lens.max()), scale=0.088,
                               partition_size=-1, num_blocks=int(kc.shape[0]))
    torch.cuda.synchronize()
    return out


def test_preempted_sequences_resume_with_bit_identical_attention(gpu):
    rng = np.random.default_rng(41)
    gen = torch.Generator().manual_seed(41)
    B, hq, hkv, d, bs = 12, 32, 8, 128, 16
    lens = rng.integers(1, 600, size=B)
    need = int(sum(-(-int(L) // bs) for L in lens))
    N, H = need + 48, need
    a = gpu.BlockAllocator(N, bs, rng.permutation(N).astype(np.int32))
    a.set_swap_space(H)
    for i in range(B):
        a.create(i, int(lens[i]))
    a.fork(0, 100)                       # 0 and 100 share every block
    a.fork(3, 101)
    for _ in range(5):
        a.append_slot(100)               # copy of the shared partial block, then new ones
    ids = list(range(B)) + [100, 101]
    # N(0, 1) values (arbitrary bit patterns would include NaN and Inf).
    kc = torch.randn(N, hkv, d * bs, generator=gen).to(torch.bfloat16).cuda()
    vc = torch.randn(N, hkv, d * bs, generator=gen).to(torch.bfloat16).cuda()
    q = torch.randn(len(ids), hq, d, generator=gen).to(torch.bfloat16).cuda()
    maxb = max(-(-a.seq_len(i) // bs) for i in ids)
    tabs0, lens0 = a.build_block_tables(ids, maxb)
    out0 = _decode(gpu, q, kc, vc, tabs0, lens0, hkv, bs)
    assert torch.isfinite(out0.float()).all()

    group = [0, 100, 5, 7]
    hk = torch.zeros((H, hkv, d * bs), dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    kw = dict(num_kv_heads=hkv, head_dim=d, block_size=bs)
    pairs = a.swap_out(group)
    shared = len(set(a.block_table(0)) & set(a.block_table(100)))
    assert shared > 0 and all(a.host_refcount(int(b)) == 2 for b in
                              set(a.block_table(0)) & set(a.block_table(100)))
    gpu.swap_blocks(hk, hv, kc, vc, to_dev(pairs), **kw)
    torch.cuda.synchronize()
    # The freed device blocks are reused and overwritten while the group is out.
    a.create(200, 300)
    freed = torch.tensor([b for b in range(N) if a.refcount(b) == 0] + a.block_table(200))
    kc[freed.cuda()] = float("nan")
    vc[freed.cuda()] = float("nan")
    a.free(200)
    back = a.swap_in([7, 100, 0, 5])
    gpu.swap_blocks(kc, vc, hk, hv, torch.from_numpy(back).pin_memory(), **kw)
    torch.cuda.synchronize()
    assert a.num_free_host() == H
    tabs1, lens1 = a.build_block_tables(ids, maxb)
    assert np.array_equal(lens1, lens0)
    moved = [ids.index(s) for s in group]
    assert not np.array_equal(tabs1[moved], tabs0[moved])
    # Sharing inside the group came back as sharing.
    k = len(a.block_table(0)) - 1
    assert a.block_table(0)[:k] == a.block_table(100)[:k]
    out1 = _decode(gpu, q, kc, vc, tabs1, lens1, hkv, bs)
    assert torch.isfinite(out1.float()).all()
    assert torch.equal(out1, out0)


def test_deep_validation_rejects_pairs_outside_the_pools(gpu, monkeypatch):
    gen = torch.Generator().manual_seed(42)
    kc, vc = _random_bf16((8, 2, 64 * 16), gen, False), _random_bf16((8, 2, 64 * 16), gen, False)
    hk, hv = _random_bf16((4, 2, 64 * 16), gen, True), _random_bf16((4, 2, 64 * 16), gen, True)
    monkeypatch.setenv("PA_VALIDATE", "1")
    for bad in ([[8, 0]], [[0, 4]], [[1, 2], [3, 2]]):
        with pytest.raises(gpu.PagedAttnError):
            gpu.swap_blocks(hk, hv, kc, vc, to_dev(np.array(bad, np.int64)), num_kv_heads=2,
                            head_dim=64, block_size=16)


def test_pageable_host_memory_is_refused_before_any_launch(gpu):
    gen = torch.Generator().manual_seed(43)
    kc, vc = _random_bf16((8, 2, 64 * 16), gen, False), _random_bf16((8, 2, 64 * 16), gen, False)
    hk = torch.zeros((4, 2, 64 * 16), dtype=torch.bfloat16)        # not pinned
    hv = torch.zeros_like(hk)
    lib = gpu.load()
    m = to_dev(np.array([[1, 2]], np.int64))
    st = lib.pa_swap_blocks(hk.data_ptr(), hv.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                            m.data_ptr(), 1, 2, 64, 16, 8, 4, gpu.PA_BF16, None)
    assert st == gpu.PA_ERR_INVALID_ARG
    assert b"pinned" in lib.pa_last_error()
    assert torch.all(hk == 0)
