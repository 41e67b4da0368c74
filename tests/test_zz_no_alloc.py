"""pa_paged_attention_decode_noalloc on the GPU, through the C ABI: the
library's own device array in place of a workspace must give exactly what
pa_paged_attention_decode_append gives with a caller's workspace (same
kernels, same split): outputs and pools bit for bit.  Two calls in a row on
the shared array, the second with a smaller input, so the second also runs
on whatever the first left there."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import TOL, max_abs_err, oracle_decode, to_dev

pytestmark = pytest.mark.gpu

BAL = -1


def _call(pa, case, ps, noalloc, fused=True, out_dtype=None):
    kc, vc = case.key_cache.clone(), case.value_cache.clone()
    out = torch.empty(case.query.shape, dtype=out_dtype or case.query.dtype, device="cuda")
    kw = dict(num_kv_heads=case.num_kv_heads, block_size=case.block_size,
              max_context_len=int(case.context_lens.max()), scale=case.scale,
              partition_size=ps, num_blocks=case.num_blocks)
    if fused:
        kw.update(new_key=case.new_key, new_value=case.new_value,
                  slot_mapping=to_dev(case.slot_mapping))
    fn = pa.paged_attention_decode_noalloc if noalloc else pa.paged_attention_decode
    fn(out, case.query, kc, vc, to_dev(case.block_tables), to_dev(case.context_lens), **kw)
    torch.cuda.synchronize()
    return out, kc, vc


@pytest.mark.parametrize("ps", [BAL, 1024])
def test_noalloc_equals_the_workspace_call_twice_in_a_row(gpu, ps):
    big = W.make_case("70b", device="cuda")           # ~43 MB (balanced) or 34 MB of scratch
    small = W.make_case("70b", device="cuda", batch=24, len_range=(1, 900))
    for case in (big, small):
        ref_out, ref_k, ref_v = _call(gpu, case, ps, noalloc=False)
        out, k, v = _call(gpu, case, ps, noalloc=True)
        assert torch.equal(out, ref_out)
        assert torch.equal(k, ref_k) and torch.equal(v, ref_v)
    ref = oracle_decode(small, pools=(W.host_array(k), W.host_array(v)))
    assert max_abs_err(out, ref) <= TOL["bf16"] + 2.0 ** -8 * float(np.abs(ref).max())


def test_noalloc_plain_decode_and_other_bodies(gpu):
    """No new tokens (the plain decode), the VALU body and fp32 pools, each
    after another call has left its contents in the shared array."""
    for name, kw in (("7b", {}), ("tiny", {}), ("long", dict(batch=2, lens=(30000, 4000)))):
        case = W.make_case(name, device="cuda", **kw)
        for fused in (False, True):
            ref_out, ref_k, ref_v = _call(gpu, case, BAL, noalloc=False, fused=fused)
            out, k, v = _call(gpu, case, BAL, noalloc=True, fused=fused)
            assert torch.equal(out, ref_out), (name, fused)
            assert torch.equal(k, ref_k) and torch.equal(v, ref_v)


def test_noalloc_refuses_sizes_beyond_its_array_before_any_launch(gpu):
    """A split whose partial rows need more than the library's array: the
    host check refuses it and nothing is written."""
    case = W.make_case("70b", device="cuda", batch=8, len_range=(100, 300))
    out = torch.full(case.query.shape, 7.0, dtype=case.query.dtype, device="cuda")
    # max_context_len sizes the fixed split: 8 sequences * 8 units * 2048
    # partitions of 16 tokens * 8 rows * 130 floats is 545 MB of partial rows.
    tab = np.zeros((case.batch, 2048), np.int32)
    tab[:, :case.block_tables.shape[1]] = case.block_tables
    with pytest.raises(gpu.PagedAttnError) as e:
        gpu.paged_attention_decode_noalloc(
            out, case.query, case.key_cache, case.value_cache, to_dev(tab),
            to_dev(case.context_lens), num_kv_heads=case.num_kv_heads, block_size=16,
            max_context_len=2048 * 16, scale=case.scale, partition_size=16,
            num_blocks=case.num_blocks)
    assert e.value.status == gpu.PA_ERR_INVALID_ARG
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
