"""paged_attention_decode_append on the GPU: one launch that writes each
sequence's new token into its slot and attends.  It must leave the pools
byte-identical to reshape_and_cache followed by paged_attention_decode, give
bit-identical outputs to that pair, and match the oracle run on the written
pools (same tolerances as the plain decode)."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import TOL, max_abs_err, to_dev

pytestmark = pytest.mark.gpu

BAL = -1


def _run(pa, case, ps, slots, fused, out_dtype=None):
    """Fresh copies of the pools, then either the fused call or write + attend."""
    kc, vc = case.key_cache.clone(), case.value_cache.clone()
    out = torch.empty(case.query.shape, dtype=out_dtype or case.query.dtype, device="cuda")
    tab, ln, sl = to_dev(case.block_tables), to_dev(case.context_lens), to_dev(slots)
    kw = dict(num_kv_heads=case.num_kv_heads, block_size=case.block_size,
              max_context_len=int(case.context_lens.max()), scale=case.scale,
              partition_size=ps, num_blocks=case.num_blocks)
    if fused:
        pa.paged_attention_decode(out, case.query, kc, vc, tab, ln, new_key=case.new_key,
                                  new_value=case.new_value, slot_mapping=sl, **kw)
    else:
        pa.reshape_and_cache(case.new_key, case.new_value, kc, vc, sl,
                             block_size=case.block_size, num_blocks=case.num_blocks)
        pa.paged_attention_decode(out, case.query, kc, vc, tab, ln, **kw)
    torch.cuda.synchronize()
    return out, kc, vc


def _oracle(case, slots, idx=None):
    kc = W.host_array(case.key_cache).copy()
    vc = W.host_array(case.value_cache).copy()
    oracle.reshape_and_cache(W.host_array(case.new_key), W.host_array(case.new_value), kc, vc,
                             slots, num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                             block_size=case.block_size, num_blocks=case.num_blocks)
    q, tab, ln = W.host_array(case.query), case.block_tables, case.context_lens
    if idx is not None:
        q, tab, ln = q[idx], tab[idx], ln[idx]
    ref = oracle.paged_attention(q, kc, vc, tab, ln, num_kv_heads=case.num_kv_heads,
                                 head_dim=case.head_dim, block_size=case.block_size,
                                 scale=case.scale, num_blocks=case.num_blocks, threads=16)
    return ref, kc, vc


def _bound(case, ref, out):
    b = TOL[case.dtype]
    return b + (2.0 ** -8 * np.abs(ref) if out.dtype == torch.bfloat16 else 0.0)


def _check_case(pa, case, ps, slots=None, out_dtype=None):
    slots = case.slot_mapping if slots is None else slots
    out_f, kc_f, vc_f = _run(pa, case, ps, slots, fused=True, out_dtype=out_dtype)
    out_u, kc_u, vc_u = _run(pa, case, ps, slots, fused=False, out_dtype=out_dtype)
    ref, kc_o, vc_o = _oracle(case, slots)
    assert W.host_array(kc_f).tobytes() == kc_o.tobytes()
    assert W.host_array(vc_f).tobytes() == vc_o.tobytes()
    assert W.host_array(kc_u).tobytes() == kc_o.tobytes()
    diff = np.abs(out_f.double().cpu().numpy() - ref)
    assert torch.isfinite(out_f.float()).all()
    assert np.all(diff <= _bound(case, ref, out_f)), float(diff.max())
    # The new token enters the same registers the cache read would fill, so
    # the arithmetic is the unfused path's, bit for bit.
    assert torch.equal(out_f, out_u)
    return out_f, out_u


# Shapes of every body and split, with context lengths that put the new
# token alone in its tile (17, 33, 1), last in a full tile (16, 32), or in
# a block past the first table chunk (1100).
CASES = [
    ("tiny", {}),                                                                 # fp32 MHA
    ("tiny", dict(num_q_heads=8, num_kv_heads=2, lens=(1, 17, 64, 129), pool=40)),  # fp32 GQA
    ("7b", dict(batch=6, lens=(1, 16, 17, 33, 1100, 255))),                       # bf16 MHA
    ("70b", dict(batch=6, lens=(1, 16, 17, 32, 33, 700))),                        # G = 8
    ("70b", dict(batch=4, lens=(1, 31, 33, 400), block_size=32)),
    ("70b", dict(batch=4, lens=(1, 63, 65, 400), block_size=64)),
    ("7b", dict(batch=3, lens=(1, 64, 300), block_size=64)),
    ("7b", dict(batch=4, len_range=(1, 200), num_q_heads=64, num_kv_heads=2)),    # G = 32
    ("7b", dict(batch=4, len_range=(1, 200), num_q_heads=24, num_kv_heads=8,
                head_dim=64)),                                                    # G = 3, d 64
    ("long", dict(batch=2, lens=(3000, 1537))),
]


@pytest.mark.parametrize("name,kw", CASES)
@pytest.mark.parametrize("ps", [0, 16, 64, BAL, -2])   # -2: PA_PARTITION_AUTO
def test_append_equals_write_then_attend(gpu, name, kw, ps):
    case = W.make_case(name, device="cuda", **kw)
    if ps > 0 and ps % case.block_size:
        pytest.skip("partition size must be a multiple of the block size")
    _check_case(gpu, case, ps)


def test_negative_slots_attend_the_cache_as_is(gpu):
    case = W.make_case("70b", device="cuda", batch=6, lens=(1, 17, 40, 64, 100, 300))
    slots = case.slot_mapping.copy()
    slots[[1, 4]] = -1
    for ps in (0, BAL):
        _check_case(gpu, case, ps, slots=slots)


def test_bf16_and_fp32_outputs(gpu):
    case = W.make_case("70b", device="cuda", batch=5, lens=(1, 17, 40, 64, 700))
    for od in (torch.float32, torch.bfloat16):
        _check_case(gpu, case, BAL, out_dtype=od)


def test_old_contents_of_the_new_slots_are_never_read(gpu):
    """NaN in the slots about to be written must not reach the outputs."""
    case = W.make_case("70b", device="cuda", batch=5, lens=(1, 17, 40, 64, 700))
    clean, _, _ = _run(gpu, case, BAL, case.slot_mapping, fused=True)
    bs, hkv, d = case.block_size, case.num_kv_heads, case.head_dim
    kc = case.key_cache.view(case.num_blocks, hkv, d // 8, bs, 8)
    vc = case.value_cache.view(case.num_blocks, hkv, d, bs)
    for s in case.slot_mapping.tolist():
        kc[s // bs, :, :, s % bs, :] = float("nan")
        vc[s // bs, :, :, s % bs] = float("nan")
    for ps in (0, 16, BAL):
        out, kcf, _ = _run(gpu, case, ps, case.slot_mapping, fused=True)
        assert torch.isfinite(out.float()).all()
        if ps == BAL:
            assert torch.equal(out, clean)


@pytest.mark.parametrize("name,batch", [("7b", 64), ("70b", 128)])
def test_more_new_tokens_than_waves(gpu, name, batch):
    """Short contexts keep the balanced grid small (a few tiles per wave), so
    each wave stores the new tokens of several (sequence, KV head) pairs
    after its pieces."""
    lens = tuple(1 + (7 * i) % 16 for i in range(batch))
    case = W.make_case(name, device="cuda", batch=batch, lens=lens)
    _check_case(gpu, case, BAL)


@pytest.mark.parametrize("name", ["7b", "70b", "long", "mixed"])
def test_full_size_steps_on_every_row(gpu, name):
    case = W.make_case(name, device="cuda")
    out, kc, vc = _run(gpu, case, BAL, case.slot_mapping, fused=True)
    ref, kc_o, vc_o = _oracle(case, case.slot_mapping)
    assert W.host_array(kc).tobytes() == kc_o.tobytes()
    assert W.host_array(vc).tobytes() == vc_o.tobytes()
    assert max_abs_err(out, ref) <= TOL[case.dtype]


def test_deep_validation_rejects_a_slot_off_the_last_position(gpu, monkeypatch):
    case = W.make_case("70b", device="cuda", batch=3, lens=(20, 40, 60))
    monkeypatch.setenv("PA_VALIDATE", "1")
    _run(gpu, case, BAL, case.slot_mapping, fused=True)        # consistent slots pass
    bad = case.slot_mapping.copy()
    bad[1] -= 1                                                # position L - 2
    with pytest.raises(gpu.PagedAttnError) as e:
        _run(gpu, case, BAL, bad, fused=True)
    assert e.value.status == gpu.PA_ERR_INVALID_ARG
