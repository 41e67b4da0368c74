"""Seeded random configurations across the parameter space, each checked
against the oracle: K/V dtype, head_dim, block size, KV heads and group size,
batch, lengths (empty and ragged sequences among them), split mode (auto too), output
dtype, reused-block loads and the in-launch cache write.  Every case prints
its configuration first, so a failure names it."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import TOL, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 96


def _config(k):
    rng = np.random.default_rng(9000 + k)
    bs = int(rng.choice([16, 32, 64]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    batch = int(rng.integers(1, 25))
    if hkv * group > 64:
        batch = min(batch, 6)
    max_len = int(rng.choice([16, 100, 700, 3000]))
    lens = rng.integers(0, max_len + 1, size=batch)
    lens[rng.random(batch) < 0.15] = 0
    if lens.max() == 0:
        lens[0] = 1
    ps = int(rng.choice([-1, -1, -2, 0, bs, 2 * bs, 512]))   # -2: PA_PARTITION_AUTO
    return dict(fp32=bool(rng.random() < 0.3), head_dim=int(rng.choice([64, 128])),
                block_size=bs, num_kv_heads=hkv, num_q_heads=hkv * group,
                lens=tuple(int(x) for x in lens), partition_size=ps,
                out_fp32=bool(rng.random() < 0.3), reused=bool(rng.random() < 0.25),
                append=bool(rng.random() < 0.5), seed=9000 + k)


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_configuration_matches_the_oracle(gpu, k):
    cfg = _config(k)
    print("case", k, cfg, flush=True)
    case = W.make_case("tiny" if cfg["fp32"] else "7b", device="cuda", lens=cfg["lens"],
                       batch=len(cfg["lens"]), block_size=cfg["block_size"], seed=cfg["seed"],
                       num_q_heads=cfg["num_q_heads"], num_kv_heads=cfg["num_kv_heads"],
                       head_dim=cfg["head_dim"], pool="1.5x")
    out_dtype = torch.float32 if cfg["out_fp32"] else case.query.dtype
    out = torch.empty(case.query.shape, dtype=out_dtype, device="cuda")
    kc, vc = case.key_cache.clone(), case.value_cache.clone()
    news = dict(new_key=case.new_key, new_value=case.new_value,
                slot_mapping=to_dev(case.slot_mapping)) if cfg["append"] else {}
    gpu.paged_attention_decode(out, case.query, kc, vc, to_dev(case.block_tables),
                               to_dev(case.context_lens), num_kv_heads=case.num_kv_heads,
                               block_size=case.block_size,
                               max_context_len=int(case.context_lens.max()), scale=case.scale,
                               partition_size=cfg["partition_size"], num_blocks=case.num_blocks,
                               kv_reused=cfg["reused"], **news)
    torch.cuda.synchronize()
    kp, vp = W.host_array(case.key_cache).copy(), W.host_array(case.value_cache).copy()
    if cfg["append"]:
        oracle.reshape_and_cache(W.host_array(case.new_key), W.host_array(case.new_value), kp, vp,
                                 case.slot_mapping, num_kv_heads=case.num_kv_heads,
                                 head_dim=case.head_dim, block_size=case.block_size,
                                 num_blocks=case.num_blocks)
    assert W.host_array(kc).tobytes() == kp.tobytes()
    assert W.host_array(vc).tobytes() == vp.tobytes()
    ref = oracle.paged_attention(W.host_array(case.query), kp, vp, case.block_tables,
                                 case.context_lens, num_kv_heads=case.num_kv_heads,
                                 head_dim=case.head_dim, block_size=case.block_size,
                                 scale=case.scale, num_blocks=case.num_blocks, threads=16)
    got = out.double().cpu().numpy()
    bound = TOL[case.dtype] + (2.0 ** -8 * np.abs(ref) if out_dtype == torch.bfloat16 else 0.0)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert np.all(err <= bound), "max err %.3g" % float(err.max())
