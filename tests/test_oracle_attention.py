"""Pins of the attention oracle against things other than itself.

* brute force: unpaged softmax attention on the contiguous K/V before they
  were scattered, by two library routes (torch's fp64 CPU
  scaled_dot_product_attention, and scipy's softmax with numpy products);
* invariance under a random permutation of the physical blocks;
* identical outputs for a sequence whose prefix blocks are shared and one
  holding private copies of the same contents;
* closed forms: one token, equal keys, zero scale, one dominant logit, a
  hand-worked two-token example, V -> aV + b, a common shift of all keys.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from tests import pool_layout as pl

RTOL_BRUTE = 1e-12


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bf16_values(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def _random_case(rng, B, Hq, Hkv, d, Bs, dtype, max_len=100, lens=None, spare=3):
    """Contiguous per-sequence K/V and q, scattered into a permuted pool."""
    lens = list(rng.integers(1, max_len + 1, size=B)) if lens is None else list(lens)
    nbs = [-(-int(L) // Bs) for L in lens]
    N = sum(nbs) + spare
    perm = rng.permutation(N).astype(np.int32)
    width = max(1, max(nbs))
    tables = np.zeros((B, width), dtype=np.int32)
    pos = 0
    for i, n in enumerate(nbs):
        tables[i, :n] = perm[pos:pos + n]
        pos += n
    seq_k = [rng.standard_normal((int(L), Hkv, d)).astype(np.float32) for L in lens]
    seq_v = [rng.standard_normal((int(L), Hkv, d)).astype(np.float32) for L in lens]
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    if dtype == "bf16":
        seq_k = [_bf16_bits(k) for k in seq_k]
        seq_v = [_bf16_bits(v) for v in seq_v]
        q = _bf16_bits(q)
        kp, vp = pl.empty_pools(N, Hkv, d, Bs, np.uint16)
    else:
        kp, vp = pl.empty_pools(N, Hkv, d, Bs, np.float32)
    pl.scatter_sequences(kp, vp, tables, seq_k, seq_v, Bs)
    return dict(q=q, kp=kp, vp=vp, tables=tables, lens=np.asarray(lens, dtype=np.int32),
                seq_k=seq_k, seq_v=seq_v, N=N, Hkv=Hkv, d=d, Bs=Bs, dtype=dtype)


def _run_oracle(c, scale, threads=1, tables=None, kp=None, vp=None, q=None):
    return oracle.paged_attention(
        c["q"] if q is None else q, c["kp"] if kp is None else kp,
        c["vp"] if vp is None else vp, c["tables"] if tables is None else tables, c["lens"],
        num_kv_heads=c["Hkv"], head_dim=c["d"], block_size=c["Bs"], scale=scale,
        num_blocks=c["N"], threads=threads)


def _as_f64(c, a):
    return _bf16_values(a) if c["dtype"] == "bf16" else a.astype(np.float64)


def _brute_sdpa(c, scale):
    """torch fp64 CPU scaled_dot_product_attention per sequence (unpaged)."""
    q = _as_f64(c, c["q"])
    B, Hq, d = q.shape
    G = Hq // c["Hkv"]
    out = np.zeros((B, Hq, d))
    for i in range(B):
        k = torch.from_numpy(_as_f64(c, c["seq_k"][i])).permute(1, 0, 2)   # [Hkv, L, d]
        v = torch.from_numpy(_as_f64(c, c["seq_v"][i])).permute(1, 0, 2)
        k = k.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        v = v.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        qq = torch.from_numpy(q[i]).reshape(1, Hq, 1, d)
        o = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=scale)
        out[i] = o.reshape(Hq, d).numpy()
    return out


def _brute_scipy(c, scale):
    """Textbook softmax(scale q K^T) V with scipy's softmax, per query head."""
    q = _as_f64(c, c["q"])
    B, Hq, d = q.shape
    G = Hq // c["Hkv"]
    out = np.zeros((B, Hq, d))
    for i in range(B):
        K = _as_f64(c, c["seq_k"][i])
        V = _as_f64(c, c["seq_v"][i])
        for h in range(Hq):
            w = scipy.special.softmax(scale * (K[:, h // G, :] @ q[i, h]))
            out[i, h] = w @ V[:, h // G, :]
    return out


SHAPES = [
    # B, Hq, Hkv, d, Bs, dtype
    (1, 1, 1, 16, 16, "fp32"),
    (2, 4, 2, 64, 16, "fp32"),
    (16, 8, 1, 16, 16, "fp32"),
    (2, 8, 8, 64, 32, "fp32"),
    (1, 4, 4, 16, 16, "bf16"),
    (2, 8, 2, 64, 16, "bf16"),
    (16, 8, 8, 16, 32, "bf16"),
    (2, 16, 2, 128, 16, "bf16"),
]


@pytest.mark.parametrize("B,Hq,Hkv,d,Bs,dtype", SHAPES)
def test_oracle_matches_unpaged_brute_force(B, Hq, Hkv, d, Bs, dtype):
    rng = np.random.default_rng(1000 + B * 7 + Hq * 3 + d + Bs)
    c = _random_case(rng, B, Hq, Hkv, d, Bs, dtype)
    scale = 1.0 / math.sqrt(d)
    got = _run_oracle(c, scale, threads=3)
    np.testing.assert_allclose(got, _brute_sdpa(c, scale), rtol=0, atol=RTOL_BRUTE)
    np.testing.assert_allclose(got, _brute_scipy(c, scale), rtol=0, atol=RTOL_BRUTE)


def test_oracle_tiny_workload_lengths_against_brute_force():
    """The tiny workload's shape: lengths {17,33,64,100}, 8/8 heads, d 64, Bs 16, fp32."""
    rng = np.random.default_rng(305)
    c = _random_case(rng, 4, 8, 8, 64, 16, "fp32", lens=[17, 33, 64, 100], spare=48)
    got = _run_oracle(c, 1 / 8)
    np.testing.assert_allclose(got, _brute_sdpa(c, 1 / 8), rtol=0, atol=RTOL_BRUTE)


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(7)
    c = _random_case(rng, 9, 8, 2, 64, 16, "bf16")
    a = _run_oracle(c, 0.125, threads=1)
    b = _run_oracle(c, 0.125, threads=5)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_permutation_of_physical_blocks_is_invisible(dtype):
    rng = np.random.default_rng(11)
    c = _random_case(rng, 6, 8, 4, 64, 16, dtype, spare=9)
    base = _run_oracle(c, 0.125)
    pi = rng.permutation(c["N"])
    kp2 = np.empty_like(c["kp"]); kp2[pi] = c["kp"]
    vp2 = np.empty_like(c["vp"]); vp2[pi] = c["vp"]
    tab2 = pi[c["tables"]].astype(np.int32)
    moved = _run_oracle(c, 0.125, tables=tab2, kp=kp2, vp=vp2)
    assert np.array_equal(base, moved)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_shared_prefix_blocks_give_identical_outputs(dtype):
    """Seq 0 holds private copies of a 3-block prefix; seq 1 points at seq 2's blocks."""
    rng = np.random.default_rng(12)
    Hq, Hkv, d, Bs = 8, 2, 64, 16
    P, tail_a, tail_c = 3 * Bs, 21, 9
    c = _random_case(rng, 3, Hq, Hkv, d, Bs, dtype, lens=[P + tail_a, P + tail_a, P + tail_c])
    # Make seq 1 a logical copy of seq 0 (same q, same tail, same prefix contents)
    # and have its prefix share seq 2's physical blocks, whose prefix content we
    # overwrite with seq 0's prefix.
    q = c["q"].copy(); q[1] = q[0]
    tab = c["tables"].copy()
    tab[1, :3] = tab[2, :3]
    kp, vp = c["kp"].copy(), c["vp"].copy()
    kp[tab[2, :3]] = kp[c["tables"][0, :3]]
    vp[tab[2, :3]] = vp[c["tables"][0, :3]]
    kp[tab[1, 3:5]] = kp[c["tables"][0, 3:5]]
    vp[tab[1, 3:5]] = vp[c["tables"][0, 3:5]]
    out = _run_oracle(c, 0.125, tables=tab, kp=kp, vp=vp, q=q)
    assert np.array_equal(out[0], out[1])
    # Seq 2 reads the overwritten prefix: it must equal brute force on that content.
    k2, v2 = pl.gather_sequence(kp, vp, tab[2], P + tail_c, Bs)
    c2 = dict(c, q=q[2:3], seq_k=[k2], seq_v=[v2])
    np.testing.assert_allclose(out[2:3], _brute_sdpa(c2, 0.125), rtol=0, atol=RTOL_BRUTE)


def _single_seq(rng, L, d=16, Hq=2, Hkv=1, Bs=16, k=None, v=None, q=None):
    k = rng.standard_normal((L, Hkv, d)).astype(np.float32) if k is None else k
    v = rng.standard_normal((L, Hkv, d)).astype(np.float32) if v is None else v
    q = rng.standard_normal((1, Hq, d)).astype(np.float32) if q is None else q
    nb = -(-L // Bs)
    N = nb + 4
    tables = rng.permutation(N)[:nb].astype(np.int32).reshape(1, nb)
    kp, vp = pl.empty_pools(N, Hkv, d, Bs, np.float32, fill=np.nan)
    pl.scatter_sequences(kp, vp, tables, [k], [v], Bs, fill=np.nan)
    return dict(q=q, kp=kp, vp=vp, tables=tables, lens=np.array([L], np.int32), seq_k=[k],
                seq_v=[v], N=N, Hkv=Hkv, d=d, Bs=Bs, dtype="fp32")


def test_one_token_returns_its_value_exactly():
    rng = np.random.default_rng(13)
    c = _single_seq(rng, 1)
    out = _run_oracle(c, 0.25)
    for h in range(2):
        assert np.array_equal(out[0, h], c["seq_v"][0][0, 0].astype(np.float64))


def test_equal_keys_give_the_mean_of_values():
    rng = np.random.default_rng(14)
    L = 37
    k = np.repeat(rng.standard_normal((1, 1, 16)).astype(np.float32), L, axis=0)
    c = _single_seq(rng, L, k=k)
    out = _run_oracle(c, 0.25)
    mean = c["seq_v"][0][:, 0, :].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[0, 0], mean, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[0, 1], mean, rtol=0, atol=1e-13)


def test_zero_scale_gives_the_mean_of_values():
    rng = np.random.default_rng(15)
    c = _single_seq(rng, 45)
    out = _run_oracle(c, 0.0)
    mean = c["seq_v"][0][:, 0, :].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[0, 1], mean, rtol=0, atol=1e-13)


def test_dominant_logit_selects_its_value_without_overflow():
    """One logit ~1e4 above the rest: exp of the others underflows to 0 exactly.

    Without subtracting the maximum the weights would overflow to inf and the
    output would be NaN.
    """
    rng = np.random.default_rng(16)
    L, d = 50, 16
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((L, 1, d)).astype(np.float32)
    star = 23
    k[star, 0] = q[0, 0] * np.float32(1e4 / float(q[0, 0] @ q[0, 0]))
    c = _single_seq(rng, L, Hq=1, k=k, q=q)
    out = _run_oracle(c, 1.0)
    assert np.array_equal(out[0, 0], c["seq_v"][0][star, 0].astype(np.float64))


def test_hand_worked_two_token_example():
    """q=(1,0,0,0), k0=(ln 3,0,0,0), k1=0, scale 1: weights 3/4 and 1/4.

    v0=(1,2,0,0), v1=(5,-2,0,0) -> out = (0.75+1.25, 1.5-0.5, 0, 0) = (2, 1, 0, 0).
    The two tokens sit in two different physical blocks of size 1.
    """
    d = 4
    q = np.array([[[1, 0, 0, 0]]], np.float32)
    k = np.zeros((2, 1, d), np.float32); k[0, 0, 0] = np.float32(math.log(3.0))
    v = np.array([[[1, 2, 0, 0]], [[5, -2, 0, 0]]], np.float32)
    kp, vp = pl.empty_pools(8, 1, d, 1, np.float32, fill=np.nan)
    tables = np.array([[5, 2]], np.int32)
    pl.scatter_sequences(kp, vp, tables, [k], [v], 1)
    out = oracle.paged_attention(q, kp, vp, tables, np.array([2], np.int32), num_kv_heads=1,
                                 head_dim=d, block_size=1, scale=1.0, num_blocks=8)
    np.testing.assert_allclose(out[0, 0], [2.0, 1.0, 0.0, 0.0], rtol=0, atol=1e-7)


def test_affine_map_of_values_maps_the_output():
    """V -> a V + b gives out -> a out + b (weights sum to one)."""
    rng = np.random.default_rng(17)
    L = 70
    # Values on a 1/256 grid so that a V + b is exact in fp32.
    v = (np.round(rng.standard_normal((L, 1, 16)) * 256) / 256).astype(np.float32)
    c = _single_seq(rng, L, v=v)
    a, b = np.float32(0.5), np.float32(3.0)
    c2 = _single_seq(rng, L, k=c["seq_k"][0], v=a * c["seq_v"][0] + b, q=c["q"])
    o1 = _run_oracle(c, 0.25)
    o2 = _run_oracle(c2, 0.25)
    np.testing.assert_allclose(o2, 0.5 * o1 + 3.0, rtol=0, atol=1e-12)


def test_common_shift_of_all_keys_leaves_output_unchanged():
    """k_t -> k_t + u adds scale <q,u> to every logit, which softmax cancels."""
    rng = np.random.default_rng(18)
    L = 33
    # Keys on a 1/256 grid so that k + u is exact in fp32.
    k = (np.round(rng.standard_normal((L, 1, 16)) * 256) / 256).astype(np.float32)
    c = _single_seq(rng, L, Hq=1, k=k)
    u = np.zeros((1, 1, 16), np.float32); u[0, 0, 3] = 2.0
    c2 = _single_seq(rng, L, Hq=1, k=c["seq_k"][0] + u, v=c["seq_v"][0], q=c["q"])
    np.testing.assert_allclose(_run_oracle(c2, 0.25), _run_oracle(c, 0.25), rtol=0, atol=1e-12)


def test_zero_length_rows_are_zero_and_unfilled_slots_are_not_read():
    rng = np.random.default_rng(19)
    c = _random_case(rng, 3, 4, 2, 16, 16, "fp32", lens=[5, 1, 20])
    # Poison every slot past each sequence's length and every unused block.
    kp, vp = pl.empty_pools(c["N"], 2, 16, 16, np.float32, fill=np.nan)
    pl.scatter_sequences(kp, vp, c["tables"], c["seq_k"], c["seq_v"], 16, fill=np.nan)
    lens = c["lens"].copy(); lens[1] = 0
    out = oracle.paged_attention(c["q"], kp, vp, c["tables"], lens, num_kv_heads=2, head_dim=16,
                                 block_size=16, scale=0.25, num_blocks=c["N"])
    assert np.all(out[1] == 0.0)
    assert np.all(np.isfinite(out))
    ref = _brute_sdpa(dict(c, kp=kp, vp=vp), 0.25)
    np.testing.assert_allclose(out[[0, 2]], ref[[0, 2]], rtol=0, atol=RTOL_BRUTE)


def test_out_of_range_block_is_rejected():
    rng = np.random.default_rng(20)
    c = _random_case(rng, 1, 2, 1, 16, 16, "fp32", lens=[20])
    bad = c["tables"].copy(); bad[0, 1] = c["N"]
    with pytest.raises(ValueError):
        _run_oracle(c, 0.25, tables=bad)
