"""The seeded generators are deterministic and build the stated structure."""
import math

import numpy as np
import pytest
import torch

import workloads as W


def test_seeds_follow_workload_order():
    assert [W.seed_for(n) for n in W.CONFIG_ORDER] == [305, 306, 307, 308, 309]


@pytest.mark.parametrize("name", ["tiny", "7b", "70b", "long"])
def test_structure_is_deterministic_and_consistent(name):
    a = W.case_structure(name)
    b = W.case_structure(name)
    assert np.array_equal(a.lengths, b.lengths) and np.array_equal(a.perm, b.perm)
    assert np.array_equal(a.tables, b.tables) and np.array_equal(a.slots, b.slots)
    cfg = W.CONFIGS[name]
    bs = a.block_size
    nb = [-(-int(L) // bs) for L in a.lengths]
    assert sorted(a.perm.tolist()) == list(range(a.num_blocks))
    # Sequences take consecutive runs of the permutation, in order.
    flat = np.concatenate([a.tables[i, :n] for i, n in enumerate(nb)])
    assert np.array_equal(flat, a.perm[:sum(nb)])
    if "len_range" in cfg:
        lo, hi = cfg["len_range"]
        assert a.lengths.min() >= lo and a.lengths.max() <= hi and len(a.lengths) == cfg["batch"]
    else:
        assert tuple(a.lengths) == tuple(cfg["lens"])
    if cfg["pool"] == "1.5x":
        assert a.num_blocks == math.ceil(1.5 * sum(nb))
    elif cfg["pool"] == "exact":
        assert a.num_blocks == sum(nb)
    else:
        assert a.num_blocks == cfg["pool"]
    # The new token sits at position L-1 of each sequence.
    for i, L in enumerate(a.lengths):
        p = int(L) - 1
        assert a.slots[i] == a.tables[i, p // bs] * bs + p % bs


def test_long_workload_with_block_size_32():
    a = W.case_structure("long", block_size=32)
    assert a.num_blocks == 8 * 32768 // 32 and a.tables.shape == (8, 1024)


def test_tensors_are_deterministic_per_seed():
    a = W.make_case("tiny")
    b = W.make_case("tiny")
    for f in ("query", "key_cache", "value_cache", "new_key", "new_value"):
        assert torch.equal(getattr(a, f), getattr(b, f))
    c = W.make_case("tiny", seed=1)
    assert not torch.equal(a.query, c.query)
    assert a.key_cache.shape == (64, 8, 16 * 64) and a.query.dtype == torch.float32


def test_bf16_tensors_are_rne_narrowings_of_fp32_draws():
    a = W.make_case("7b", batch=2, len_range=(20, 40))
    gen = torch.Generator().manual_seed(a.seed)
    q32 = torch.randn(2, 32, 128, generator=gen)
    assert a.query.dtype == torch.bfloat16 and torch.equal(a.query, q32.to(torch.bfloat16))


def test_shared_plan_structure():
    p = W.shared_plan()
    assert p.batch == 64 and p.prompt == 4000 and p.block_size == 16
    assert p.tails.min() >= 0 and p.tails.max() <= 512
    needed = 250 + int(sum(-(-int(t) // 16) + 1 for t in p.tails))
    assert p.num_blocks == math.ceil(1.5 * needed)
    assert sorted(p.perm.tolist()) == list(range(p.num_blocks))


def test_mixed_workload_has_one_long_context():
    """The 70B shape with one 131,072-token context at a seeded position:
    seeded after the five workloads, the other 255 lengths in [128, 4096],
    exactly the blocks needed."""
    st = W.case_structure("mixed")
    assert W.seed_for("mixed") == 310
    L = st.lengths
    assert L.shape == (256,) and (L == 131072).sum() == 1
    others = L[L != 131072]
    assert others.min() >= 128 and others.max() <= 4096
    assert st.num_blocks == int(sum(-(-int(x) // 16) for x in L))
    again = W.case_structure("mixed")
    assert (again.lengths == L).all() and (again.perm == st.perm).all()
