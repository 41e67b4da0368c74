"""Every-layer cache calls and graph capture of the decode step on the GPU.

reshape_and_cache_layers / copy_blocks_layers must leave every layer's
pools byte-identical to the oracle's per-layer scatter and copy.  A step
captured into a HIP graph is replayed several times, with its query
refilled in place and eager work in between: every replay must equal an
eager run of the same step on the same inputs, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import TOL, max_abs_err, to_dev

pytestmark = pytest.mark.gpu


def _layers(name, n, **kw):
    """n cases with the same structure (seed) but distinct float contents."""
    cases = [W.make_case(name, device="cuda", **kw) for _ in range(n)]
    gen = torch.Generator(device="cuda").manual_seed(77)
    for c in cases[1:]:
        for t in (c.key_cache, c.value_cache, c.new_key, c.new_value):
            t.copy_(torch.randn(t.shape, generator=gen, device="cuda").to(t.dtype))
    return cases


def test_reshape_and_cache_on_every_layer_matches_the_oracle(gpu):
    cases = _layers("70b", 3, batch=9, len_range=(1, 300))
    c0 = cases[0]
    host = [(W.host_array(c.key_cache).copy(), W.host_array(c.value_cache).copy()) for c in cases]
    ptr = lambda ts: gpu.pointer_array(ts, torch.device("cuda"))
    slots = to_dev(c0.slot_mapping)
    gpu.reshape_and_cache_layers(ptr([c.new_key for c in cases]),
                                 ptr([c.new_value for c in cases]),
                                 ptr([c.key_cache for c in cases]),
                                 ptr([c.value_cache for c in cases]), slots, num_layers=3,
                                 num_kv_heads=c0.num_kv_heads, head_dim=c0.head_dim,
                                 block_size=c0.block_size, num_blocks=c0.num_blocks,
                                 dtype=c0.key_cache.dtype)
    torch.cuda.synchronize()
    for c, (kh, vh) in zip(cases, host):
        oracle.reshape_and_cache(W.host_array(c.new_key), W.host_array(c.new_value), kh, vh,
                                 c0.slot_mapping, num_kv_heads=c.num_kv_heads,
                                 head_dim=c.head_dim, block_size=c.block_size,
                                 num_blocks=c.num_blocks)
        assert W.host_array(c.key_cache).tobytes() == kh.tobytes()
        assert W.host_array(c.value_cache).tobytes() == vh.tobytes()


def test_copy_blocks_on_every_layer_matches_the_oracle(gpu):
    cases = _layers("tiny", 4)
    c0 = cases[0]
    pairs = np.array([[1, 40], [1, 41], [7, 50], [20, 63]], np.int64)
    host = [(W.host_array(c.key_cache).copy(), W.host_array(c.value_cache).copy()) for c in cases]
    ptr = lambda ts: gpu.pointer_array(ts, torch.device("cuda"))
    gpu.copy_blocks_layers(ptr([c.key_cache for c in cases]), ptr([c.value_cache for c in cases]),
                           to_dev(pairs), num_layers=4, num_kv_heads=c0.num_kv_heads,
                           head_dim=c0.head_dim, block_size=c0.block_size,
                           num_blocks=c0.num_blocks, dtype=c0.key_cache.dtype)
    torch.cuda.synchronize()
    for c, (kh, vh) in zip(cases, host):
        oracle.copy_blocks(kh, vh, pairs, num_kv_heads=c.num_kv_heads, head_dim=c.head_dim,
                           block_size=c.block_size, num_blocks=c.num_blocks)
        assert W.host_array(c.key_cache).tobytes() == kh.tobytes()
        assert W.host_array(c.value_cache).tobytes() == vh.tobytes()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("ps", [-1, 64])
def test_graph_replays_equal_eager_runs(gpu, fused, ps):
    from paged_kv_cache_305_amd.step import step_from_case
    case = W.make_case("70b", device="cuda", batch=24, len_range=(1, 1500))
    step = step_from_case(case, partition_size=ps)
    step.fused = fused
    step.capture()
    gen = torch.Generator(device="cuda").manual_seed(78)
    for r in range(4):
        q = torch.randn(step.query.shape, generator=gen, device="cuda").to(step.query.dtype)
        step.query.copy_(q)
        eager = step.run().clone()
        kc, vc = step.key_cache.clone(), step.value_cache.clone()
        torch.cuda.synchronize()
        _ = (torch.randn(1 << 20, device="cuda") * 2).sum()      # unrelated eager work
        step.out.zero_()
        got = step.replay()
        torch.cuda.synchronize()
        assert torch.equal(got, eager), r
        assert torch.equal(step.key_cache, kc) and torch.equal(step.value_cache, vc)
    idx = [0, 5, 23]
    ref = oracle.paged_attention(W.host_array(step.query)[idx], W.host_array(step.key_cache),
                                 W.host_array(step.value_cache), case.block_tables[idx],
                                 case.context_lens[idx], num_kv_heads=case.num_kv_heads,
                                 head_dim=case.head_dim, block_size=case.block_size,
                                 scale=case.scale, num_blocks=case.num_blocks, threads=16)
    assert max_abs_err(step.out[idx], ref) <= TOL["bf16"]


def test_three_layer_step_in_one_graph(gpu):
    """copy_blocks_layers + reshape_and_cache_layers + attention per layer,
    captured once: replays equal the eager sequence."""
    cases = _layers("70b", 3, batch=8, len_range=(20, 400), pool=400)
    c0 = cases[0]
    dev = torch.device("cuda")
    kp, vp = gpu.pointer_array([c.key_cache for c in cases], dev), \
        gpu.pointer_array([c.value_cache for c in cases], dev)
    nk, nv = gpu.pointer_array([c.new_key for c in cases], dev), \
        gpu.pointer_array([c.new_value for c in cases], dev)
    slots, tabs, lens = to_dev(c0.slot_mapping), to_dev(c0.block_tables), to_dev(c0.context_lens)
    # Copy between blocks no sequence uses, so every run of the step is the same.
    used = {int(b) for i, L in enumerate(c0.context_lens)
            for b in c0.block_tables[i, :-(-int(L) // c0.block_size)]}
    spare = [b for b in range(c0.num_blocks) if b not in used][:2]
    assert len(spare) == 2
    pairs = to_dev(np.array([spare], np.int64))
    outs = [torch.empty_like(c.query) for c in cases]
    ws = torch.empty(gpu.paged_attention_workspace_bytes(
        c0.batch, c0.num_q_heads, c0.num_kv_heads, c0.head_dim, int(c0.context_lens.max()), -1,
        c0.query.dtype), dtype=torch.uint8, device=dev)
    shape = dict(num_kv_heads=c0.num_kv_heads, head_dim=c0.head_dim, block_size=c0.block_size,
                 num_blocks=c0.num_blocks, dtype=c0.key_cache.dtype)

    def model_step():
        gpu.copy_blocks_layers(kp, vp, pairs, num_layers=3, **shape)
        gpu.reshape_and_cache_layers(nk, nv, kp, vp, slots, num_layers=3, **shape)
        for c, o in zip(cases, outs):
            gpu.paged_attention_decode(o, c.query, c.key_cache, c.value_cache, tabs, lens,
                                       num_kv_heads=c.num_kv_heads, block_size=c.block_size,
                                       max_context_len=int(c0.context_lens.max()),
                                       scale=c.scale, partition_size=-1, workspace=ws,
                                       num_blocks=c.num_blocks)

    model_step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        model_step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        model_step()
    for _ in range(3):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e)


@pytest.mark.parametrize("kind", ["many_short_one_long", "shared_prefix_copies"])
def test_graph_replays_of_the_segment_merge_and_in_launch_copies(gpu, kind):
    """Replays of a captured step equal eager runs when the merge uses its
    per-segment counters (reset by the main kernel inside the graph, no
    memset) and when copy-on-write runs inside the attention launch."""
    from paged_kv_cache_305_amd.step import shared_prefix_step, step_from_case
    if kind == "many_short_one_long":
        rng = np.random.default_rng(21)
        lens = tuple(int(x) for x in rng.integers(0, 65, size=299)) + (30000,)
        case = W.make_case("70b", device="cuda", batch=300, lens=lens)
        step = step_from_case(case, partition_size=-1)
    else:
        plan = W.shared_plan()
        tens = W.shared_tensors(plan, device="cuda")
        step, _ = shared_prefix_step(plan, tens, partition_size=-1, prefix=True)
        assert step.uses_fused_copy
    step.capture()
    gen = torch.Generator(device="cuda").manual_seed(79)
    for r in range(3):
        q = torch.randn(step.query.shape, generator=gen, device="cuda").to(step.query.dtype)
        step.query.copy_(q)
        eager = step.run().clone()
        kc, vc = step.key_cache.clone(), step.value_cache.clone()
        torch.cuda.synchronize()
        _ = (torch.randn(1 << 20, device="cuda") * 2).sum()      # unrelated eager work
        step.out.zero_()
        got = step.replay()
        torch.cuda.synchronize()
        assert torch.equal(got, eager), r
        assert torch.equal(step.key_cache, kc) and torch.equal(step.value_cache, vc)
