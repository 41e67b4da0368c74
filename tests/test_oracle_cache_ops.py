"""Pins of the reshape_and_cache and copy_blocks oracles.

The scatter is checked against the test-side block construction (numpy
reshapes of whole blocks): writing a sequence token by token through the
oracle must produce the same pool bytes as building its blocks directly.
The copy is checked against whole-block equality and snapshot semantics.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import pool_layout as pl


@pytest.mark.parametrize("dtype,Bs,d", [(np.float32, 16, 64), (np.uint16, 16, 128),
                                        (np.uint16, 32, 64), (np.float32, 32, 16)])
def test_token_by_token_scatter_builds_the_same_pool(dtype, Bs, d):
    rng = np.random.default_rng(31)
    Hkv, L, N = 3, 75, 9
    table = rng.permutation(N)[: -(-L // Bs)].astype(np.int32)
    if dtype == np.float32:
        k = rng.standard_normal((L, Hkv, d)).astype(np.float32)
        v = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    else:
        k = rng.integers(0, 1 << 16, size=(L, Hkv, d), dtype=np.uint16)
        v = rng.integers(0, 1 << 16, size=(L, Hkv, d), dtype=np.uint16)
    want_k, want_v = pl.empty_pools(N, Hkv, d, Bs, dtype)
    pl.scatter_sequences(want_k, want_v, table[None, :], [k], [v], Bs)
    got_k, got_v = pl.empty_pools(N, Hkv, d, Bs, dtype)
    slots = np.array([table[t // Bs] * Bs + t % Bs for t in range(L)], np.int64)
    oracle.reshape_and_cache(k, v, got_k, got_v, slots, num_kv_heads=Hkv, head_dim=d,
                             block_size=Bs, num_blocks=N)
    assert got_k.tobytes() == want_k.tobytes()
    assert got_v.tobytes() == want_v.tobytes()
    # And reading back through the test-side gather returns the tokens.
    kk, vv = pl.gather_sequence(got_k, got_v, table, L, Bs)
    assert np.array_equal(kk, k) and np.array_equal(vv, v)


def test_negative_slots_are_skipped_and_other_slots_untouched():
    rng = np.random.default_rng(32)
    N, Hkv, d, Bs = 4, 2, 16, 16
    kp = rng.standard_normal((N, Hkv, d // 4, Bs, 4)).astype(np.float32)
    vp = rng.standard_normal((N, Hkv, d, Bs)).astype(np.float32)
    k0, v0 = kp.copy(), vp.copy()
    key = rng.standard_normal((3, Hkv, d)).astype(np.float32)
    val = rng.standard_normal((3, Hkv, d)).astype(np.float32)
    slots = np.array([-1, 2 * Bs + 5, -7], np.int64)
    oracle.reshape_and_cache(key, val, kp, vp, slots, num_kv_heads=Hkv, head_dim=d,
                             block_size=Bs, num_blocks=N)
    changed_k = np.argwhere(kp != k0)
    assert set(map(tuple, changed_k[:, [0, 3]])) <= {(2, 5)}
    assert np.array_equal(kp[2, :, :, 5, :].reshape(Hkv, d), key[1])
    assert np.array_equal(vp[2, :, :, 5], val[1])
    mask = np.ones_like(vp, bool); mask[2, :, :, 5] = False
    assert np.array_equal(vp[mask], v0[mask])


def test_out_of_range_slot_is_rejected():
    kp, vp = pl.empty_pools(2, 1, 16, 16, np.float32)
    key = np.zeros((1, 1, 16), np.float32)
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(key, key, kp, vp, np.array([32], np.int64), num_kv_heads=1,
                                 head_dim=16, block_size=16, num_blocks=2)


def test_copy_blocks_copies_whole_blocks_from_a_snapshot():
    rng = np.random.default_rng(33)
    N, Hkv, d, Bs = 8, 2, 64, 16
    bits = lambda shape: rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    kp = bits((N, Hkv, d // 8, Bs, 8)); vp = bits((N, Hkv, d, Bs))
    k0, v0 = kp.copy(), vp.copy()
    pairs = np.array([[1, 4], [1, 6], [3, 0]], np.int64)   # a source repeats
    oracle.copy_blocks(kp, vp, pairs, num_kv_heads=Hkv, head_dim=d, block_size=Bs, num_blocks=N)
    for s, t in pairs:
        assert np.array_equal(kp[t], k0[s]) and np.array_equal(vp[t], v0[s])
    for b in (1, 2, 3, 5, 7):
        assert np.array_equal(kp[b], k0[b]) and np.array_equal(vp[b], v0[b])


def test_copy_blocks_reads_sources_before_writing():
    """A chain 2->5, 5->7: block 7 gets the old contents of 5 (snapshot semantics)."""
    rng = np.random.default_rng(34)
    kp = rng.standard_normal((8, 1, 4, 16, 4)).astype(np.float32)
    vp = rng.standard_normal((8, 1, 16, 16)).astype(np.float32)
    k0 = kp.copy()
    oracle.copy_blocks(kp, vp, np.array([[2, 5], [5, 7]], np.int64), num_kv_heads=1,
                       head_dim=16, block_size=16, num_blocks=8)
    assert np.array_equal(kp[5], k0[2]) and np.array_equal(kp[7], k0[5])


def test_copy_blocks_with_no_pairs_is_a_no_op():
    kp, vp = pl.empty_pools(2, 1, 16, 16, np.float32, fill=1.0)
    oracle.copy_blocks(kp, vp, np.zeros((0, 2), np.int64), num_kv_heads=1, head_dim=16,
                       block_size=16, num_blocks=2)
    assert np.all(kp == 1.0)


def test_bf16_bits_survive_the_scatter_unchanged():
    """Bit copy: NaN payloads and signed zeros pass through untouched."""
    vals = torch.tensor([float("nan"), -0.0, 1e-40, 3.5], dtype=torch.float32).to(torch.bfloat16)
    bits = vals.view(torch.int16).numpy().view(np.uint16)
    key = np.tile(bits, 2).reshape(1, 1, 8)
    kp, vp = pl.empty_pools(1, 1, 8, 16, np.uint16)
    oracle.reshape_and_cache(key, key, kp, vp, np.array([3], np.int64), num_kv_heads=1,
                             head_dim=8, block_size=16, num_blocks=1)
    assert np.array_equal(kp[0, 0, 0, 3], key[0, 0])
    assert np.array_equal(vp[0, 0, 0, :, 3], key[0, 0])


# ---- swap_blocks (inferensys glossary, third and fifth paragraphs) -----------

def test_swap_out_and_back_in_restores_every_token_of_the_swapped_blocks():
    """Device pool -> swap pool -> a different device block: the gathered
    tokens of each moved block are unchanged, the rest of both pools too."""
    rng = np.random.default_rng(35)
    N, H, Hkv, d, Bs = 10, 6, 2, 64, 16
    bits = lambda shape: rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    kp, vp = bits((N, Hkv, d // 8, Bs, 8)), bits((N, Hkv, d, Bs))
    hk, hv = bits((H, Hkv, d // 8, Bs, 8)), bits((H, Hkv, d, Bs))
    k0, v0, hk0, hv0 = kp.copy(), vp.copy(), hk.copy(), hv.copy()
    out = np.array([[7, 0], [2, 5], [4, 1]], np.int64)          # device -> swap
    oracle.swap_blocks(hk, hv, kp, vp, out, num_kv_heads=Hkv, head_dim=d, block_size=Bs)
    back = np.array([[0, 3], [5, 9], [1, 8]], np.int64)         # swap -> new device blocks
    oracle.swap_blocks(kp, vp, hk, hv, back, num_kv_heads=Hkv, head_dim=d, block_size=Bs)
    for (dev, swp), (swp2, new) in zip(out, back):
        assert swp == swp2
        got = pl.gather_sequence(kp, vp, [new], Bs, Bs)
        want = pl.gather_sequence(k0, v0, [dev], Bs, Bs)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    untouched_dev = [b for b in range(N) if b not in (3, 9, 8)]
    assert np.array_equal(kp[untouched_dev], k0[untouched_dev])
    assert np.array_equal(hk[[2, 3, 4]], hk0[[2, 3, 4]]) and np.array_equal(hv[[2, 3]], hv0[[2, 3]])


def test_swap_within_one_pool_equals_copy_blocks():
    rng = np.random.default_rng(36)
    kp = rng.standard_normal((8, 2, 8, 32, 4)).astype(np.float32)
    vp = rng.standard_normal((8, 2, 32, 32)).astype(np.float32)
    pairs = np.array([[1, 4], [1, 6], [3, 0]], np.int64)
    a_k, a_v = kp.copy(), vp.copy()
    oracle.copy_blocks(a_k, a_v, pairs, num_kv_heads=2, head_dim=32, block_size=32, num_blocks=8)
    b_k, b_v = kp.copy(), vp.copy()
    oracle.swap_blocks(b_k, b_v, kp, vp, pairs, num_kv_heads=2, head_dim=32, block_size=32)
    assert np.array_equal(a_k, b_k) and np.array_equal(a_v, b_v)


def test_swap_rejects_blocks_outside_either_pool():
    kp, vp = pl.empty_pools(4, 1, 16, 16, np.float32)
    hk, hv = pl.empty_pools(2, 1, 16, 16, np.float32)
    for bad in ([[4, 0]], [[0, 2]], [[-1, 0]]):
        with pytest.raises(ValueError):
            oracle.swap_blocks(hk, hv, kp, vp, np.array(bad, np.int64), num_kv_heads=1,
                               head_dim=16, block_size=16)
