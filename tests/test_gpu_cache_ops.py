"""reshape_and_cache and copy_blocks on the GPU: the whole pools after the call
must equal, byte for byte, the oracle's scatter/copy applied to host copies."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes()


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("7b", dict(batch=40, len_range=(1, 100))),
    ("70b", dict(batch=30, len_range=(1, 100), block_size=32)),
    ("7b", dict(batch=30, len_range=(1, 100), head_dim=64, num_q_heads=8, num_kv_heads=8)),
    ("tiny", dict(head_dim=128, block_size=32)),
])
def test_reshape_and_cache_matches_oracle_bit_exact(gpu, name, kw):
    case = W.make_case(name, device="cuda", **kw)
    T = case.batch
    rng = np.random.default_rng(5)
    slots = rng.choice(case.num_blocks * case.block_size, size=T, replace=False).astype(np.int64)
    slots[rng.random(T) < 0.2] = -1           # skipped tokens
    kc_h, vc_h = W.host_array(case.key_cache).copy(), W.host_array(case.value_cache).copy()
    gpu.reshape_and_cache(case.new_key, case.new_value, case.key_cache, case.value_cache,
                          to_dev(slots), block_size=case.block_size)
    torch.cuda.synchronize()
    oracle.reshape_and_cache(W.host_array(case.new_key), W.host_array(case.new_value), kc_h,
                             vc_h, slots, num_kv_heads=case.num_kv_heads,
                             head_dim=case.head_dim, block_size=case.block_size,
                             num_blocks=case.num_blocks)
    assert _bytes(case.key_cache) == kc_h.tobytes()
    assert _bytes(case.value_cache) == vc_h.tobytes()


def test_reshape_and_cache_full_7b_step_tokens(gpu):
    case = W.make_case("7b", device="cuda")
    kc_h, vc_h = W.host_array(case.key_cache).copy(), W.host_array(case.value_cache).copy()
    gpu.reshape_and_cache(case.new_key, case.new_value, case.key_cache, case.value_cache,
                          to_dev(case.slot_mapping), block_size=16)
    torch.cuda.synchronize()
    oracle.reshape_and_cache(W.host_array(case.new_key), W.host_array(case.new_value), kc_h,
                             vc_h, case.slot_mapping, num_kv_heads=32, head_dim=128,
                             block_size=16, num_blocks=case.num_blocks)
    assert _bytes(case.key_cache) == kc_h.tobytes()
    assert _bytes(case.value_cache) == vc_h.tobytes()


@pytest.mark.parametrize("name,kw", [("70b", dict(batch=20, len_range=(1, 100))),
                                     ("tiny", {}),
                                     ("long", dict(batch=1, lens=(4000,), block_size=32))])
def test_copy_blocks_matches_oracle_bit_exact(gpu, name, kw):
    case = W.make_case(name, device="cuda", **kw)
    rng = np.random.default_rng(9)
    blocks = rng.permutation(case.num_blocks)
    n = min(12, case.num_blocks // 3)
    srcs = blocks[:n // 2]
    dsts = blocks[n // 2: n // 2 + n]
    pairs = np.stack([np.resize(srcs, len(dsts)), dsts], axis=1).astype(np.int64)  # srcs repeat
    kc_h, vc_h = W.host_array(case.key_cache).copy(), W.host_array(case.value_cache).copy()
    gpu.copy_blocks(case.key_cache, case.value_cache, to_dev(pairs),
                    num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                    block_size=case.block_size)
    torch.cuda.synchronize()
    oracle.copy_blocks(kc_h, vc_h, pairs, num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                       block_size=case.block_size, num_blocks=case.num_blocks)
    assert _bytes(case.key_cache) == kc_h.tobytes()
    assert _bytes(case.value_cache) == vc_h.tobytes()


def test_copy_blocks_with_no_pairs_changes_nothing(gpu):
    case = W.make_case("tiny", device="cuda")
    before = _bytes(case.key_cache)
    gpu.copy_blocks(case.key_cache, case.value_cache, torch.zeros((0, 2), dtype=torch.int64,
                                                                  device="cuda"),
                    num_kv_heads=8, head_dim=64, block_size=16)
    torch.cuda.synchronize()
    assert _bytes(case.key_cache) == before


def test_deep_validation_rejects_bad_slots_and_pairs(gpu, monkeypatch):
    case = W.make_case("tiny", device="cuda")
    monkeypatch.setenv("PA_VALIDATE", "1")
    before = _bytes(case.key_cache)
    for slots in ([3, 3, -1, 5], [0, 1, 2, 64 * 16]):
        with pytest.raises(gpu.PagedAttnError) as e:
            gpu.reshape_and_cache(case.new_key, case.new_value, case.key_cache, case.value_cache,
                                  to_dev(np.array(slots, np.int64)), block_size=16)
        assert e.value.status == gpu.PA_ERR_INVALID_ARG
    for pairs in ([[1, 2], [3, 2]], [[1, 2], [2, 5]], [[1, 64]]):
        with pytest.raises(gpu.PagedAttnError):
            gpu.copy_blocks(case.key_cache, case.value_cache, to_dev(np.array(pairs, np.int64)),
                            num_kv_heads=8, head_dim=64, block_size=16)
    torch.cuda.synchronize()
    assert _bytes(case.key_cache) == before
