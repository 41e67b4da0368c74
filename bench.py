#!/usr/bin/env python3
"""Benchmark one decode step of the paged KV cache on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the host block allocator reserves each sequence's slot (copy-on-write pairs
where a shared block is written; done once, outside the timed region), then
on the GPU copy_blocks on those pairs, and the attention over all cached
tokens (main kernel, plus the log-sum-exp merge when a sequence spans
several pieces).  Each sequence's new token is written into its slot either
by that launch or by reshape_and_cache just before it (--cache-write; by
default the launch writes).

The default run times the 70B-shaped GQA step (the headline line) and, in
the same process, the 7B-shaped, long-context (block sizes 16 and 32),
shared-prefix and tiny steps, each reported under "workloads" with its own
timing, roofline and parity.  It also measures the GPU's streaming-read and
4 KiB-block gather ceilings (libpaprobe.so), so every kernel rate is given
as a fraction of the nominal 8 TB/s and of what the memory system delivers.

Timing: W warm-up steps, then K timed steps.  Before each step a 1 GiB
buffer is read to evict the L2s and the Infinity Cache (outside the
events); reading leaves only clean lines behind, so no write-back of the
flush competes with the step.  Each step is bracketed by HIP events on the
stream the kernels run on.  A second pass of K steps brackets the main
attention kernel with its own pair of events, recorded by the library right
around its launch (kept out of the first pass: events inside a step
lengthen it), and the end of the step with a third.

Parity: after the timed steps, every output row of the step is compared
with the CPU oracle run on host copies of the same inputs, and the pools
with the oracle's copy-on-write copies and token writes applied to a
snapshot taken before the first step (bit for bit).

Output: one JSON line (rank 0).  value = KV bytes read by attention per
step / mean step time, in GB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak, 8 TB/s
ROOT = os.path.dirname(os.path.abspath(__file__))

WORKLOADS = {
    "tiny": "tiny paged decode: 4 seqs L={17,33,64,100}, 8/8 heads, d 64, Bs 16, fp32",
    "7b": "Llama-2-7B-shaped decode: batch 64, 32/32 heads, d 128, bf16, Bs 16, L~U[512,2048]",
    "70b": "70B-shaped GQA decode: batch 256, 64/8 heads, d 128, bf16, Bs 16, L~U[128,4096]",
    "shared": "shared-prefix sampling: 64 seqs x (4000-token shared prompt + tail U[0,512]), "
              "32/8 heads, d 128, bf16, Bs 16, CoW step",
    "long": "long-context split-K: batch 8, L=32768, 32/8 heads, d 128, bf16, Bs 16",
    "long32": "long-context split-K: batch 8, L=32768, 32/8 heads, d 128, bf16, Bs 32",
    "mixed": "70B-shaped GQA decode with one long context: batch 256, 64/8 heads, d 128, bf16, "
             "Bs 16, 255 x L~U[128,4096] + one L=131072",
    "swap": "preemption swap of the 7B-shaped step's blocks: GPU pool <-> pinned host pool "
            "(swap_blocks), both directions",
    "cacheops": "the cache kernels on their own: reshape_and_cache of the 7B- and 70B-shaped "
                "steps' new tokens, copy_blocks of the shared-prefix step's copy-on-write pairs",
}
HOST_LINK_PEAK_GBS = 64.0   # PCIe Gen5 x16, one direction


MODEL_LAYERS = {"7b": 32, "70b": 80, "mixed": 80}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def build_step(name, ps, device, block_size=None, table_order="random", prefix=True, batch=None):
    import workloads as W
    from paged_kv_cache_305_amd.step import shared_prefix_step, step_from_case
    if name == "shared":
        if table_order != "random":
            raise SystemExit("the shared-prefix tables come from the allocator")
        plan = W.shared_plan(block_size=block_size, batch=batch)
        tens = W.shared_tensors(plan, device=device)
        step, rec = shared_prefix_step(plan, tens, partition_size=ps, prefix=prefix)
        lens = rec["lens"].astype(np.int64)
        return step, lens, dict(seed=plan.seed, cow_pairs=int(rec["pairs"].shape[0]),
                                num_blocks=plan.num_blocks, block_size=plan.block_size)
    base = "long" if name == "long32" else name
    bs = block_size or (32 if name == "long32" else None)
    over = dict(block_size=bs) if bs else {}
    if batch:
        over["batch"] = batch
    case = W.make_case(base, device=device, **over)
    if table_order == "identity":
        # Contiguous storage: each sequence's blocks are consecutive physical
        # blocks, sequences one after another.
        case.block_tables = W.tables_from_perm(case.context_lens,
                                               np.arange(case.num_blocks, dtype=np.int32),
                                               case.block_size)
        case.slot_mapping = W.slots_at(case.context_lens, case.block_tables, case.block_size)
    step = step_from_case(case, partition_size=ps)
    return step, case.context_lens.astype(np.int64), dict(
        seed=case.seed, num_blocks=case.num_blocks, block_size=case.block_size,
        table_order=table_order)


def unique_kv_tokens(step, lens):
    """Cached token slots the attention must read at least once: a physical
    block shared by several sequences counts once, with the most tokens any
    of them uses."""
    tabs = step.block_tables.cpu().numpy()
    used = {}
    bs = step.block_size
    for i, L in enumerate(lens.tolist()):
        nb = -(-int(L) // bs)
        for j in range(nb):
            b = int(tabs[i, j])
            used[b] = max(used.get(b, 0), min(bs, int(L) - j * bs))
    return sum(used.values())


def block_waste(step, lens):
    """Internal fragmentation of the step's cache: slots allocated in the
    distinct blocks the tables reference, and the share of them no token
    fills (each sequence wastes at most block_size - 1 slots of its last
    block)."""
    used = unique_kv_tokens(step, lens)
    tabs = step.block_tables.cpu().numpy()
    blocks = set()
    for i, L in enumerate(lens.tolist()):
        blocks.update(int(b) for b in tabs[i, :-(-int(L) // step.block_size)])
    allocated = len(blocks) * step.block_size
    return dict(kv_slots_allocated=allocated, kv_slots_used=used,
                kv_block_waste_frac=round(1.0 - used / allocated, 5) if allocated else 0.0)


# Longest context each workload reserves when storage is one contiguous
# max-length region per sequence (the prior allocation scheme the pages
# compare against): the upper end of its length distribution.
MAX_CONTEXT = {"7b": 2048, "70b": 4096, "long": 32768, "shared": 4000 + 512 + 1,
               "mixed": 131072}


def waste_report(block_sizes=(8, 16, 32, 64)):
    """KV-cache internal waste of each workload's step through the block
    allocator, per block size, next to contiguous max-length reservation
    (note-023 Key results and Concepts; inferensys glossary, first
    paragraph; crackai.dev, Why It Matters).  Host only."""
    import workloads as W
    import paged_kv_cache_305_amd as pa
    from paged_kv_cache_305_amd.step import build_shared_prefix_state
    rows = []
    for name in ("7b", "70b", "shared", "long"):
        for bs in block_sizes:
            if name == "shared":
                plan = W.shared_plan(block_size=bs)
                a = build_shared_prefix_state(plan)
                lens = [plan.prompt + int(t) for t in plan.tails]
                used = plan.prompt + int(sum(plan.tails))          # distinct tokens stored
                total = plan.num_blocks
            else:
                st = W.case_structure(name, block_size=bs)
                lens = [int(L) for L in st.lengths]
                total = int(sum(-(-L // bs) for L in lens))
                a = pa.BlockAllocator(total, bs)
                for i, L in enumerate(lens):
                    a.create(i, L)
                used = int(sum(lens))
            allocated = (total - a.num_free()) * bs
            reserved = len(lens) * MAX_CONTEXT[name]
            rows.append(dict(workload=name, block_size=bs, sequences=len(lens),
                             tokens_used=used, slots_allocated=allocated,
                             paged_waste=round(1 - used / allocated, 5),
                             contiguous_reserved_slots=reserved,
                             contiguous_waste=round(1 - sum(lens) / reserved, 5),
                             paged_over_contiguous_memory=round(allocated / reserved, 5)))
            a.close()
    return rows


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def algorithmic_bytes(step, lens):
    """(logical KV bytes, bytes the attention launch must move).

    Logical: every sequence's K and V for every KV head, as the op consumes
    them.  Launch: each distinct cached token once (K and V), q in, out
    back, the used table entries and the lengths."""
    B, hq, d = step.query.shape
    esz = step.query.element_size()
    per_token = step.num_kv_heads * d * 2 * esz
    kv = int(lens.sum()) * per_token
    qo = B * hq * d * (esz + step.out.element_size())
    tables = 4 * int(np.sum(-(-lens // step.block_size))) + 4 * B
    return kv, unique_kv_tokens(step, lens) * per_token + qo + tables


def kernel_source_digest():
    """Digest of the device sources with comments and blank space removed:
    it changes when the kernels' code changes, not when their comments do."""
    import re
    h = hashlib.sha256()
    for f in ("pa_decode.hip", "pa_cache.hip", "pa_internal.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_305_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload, ps):
    """HBM bytes per main-kernel launch from the committed counter summary, or
    None when there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_ps%d.json" % (workload, ps))
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


# ---- the oracle leg: CPU baseline and parity of the timed step -------------
#
# The CPU oracle (oracle/) runs only here, after the timed region: once timed
# on a bounded sample of the step (the CPU baseline), and once over every row
# of the step to check what the GPU computed.  The timed path never calls it.

def cpu_baseline(step, lens, max_seconds, threads=None):
    """The oracle, as it stands, on this host's cores, over a bounded sample:
    consecutive sequences of the step (wrapping around the batch), in chunks
    that double while they fit, until about max_seconds of wall time.
    threads: default min(16, cores of this host)."""
    import oracle
    import workloads as W
    if threads is None:
        threads = max(1, min(16, os.cpu_count() or 1))
    kc = W.host_array(step.key_cache)
    vc = W.host_array(step.value_cache)
    q = W.host_array(step.query)
    tab = step.block_tables.cpu().numpy()
    ln = step.context_lens.cpu().numpy()
    B = q.shape[0]
    per_seq_bytes = lens * step.num_kv_heads * step.head_dim * 2 * step.query.element_size()
    n, spent, done_bytes, done_seqs, start = 1, 0.0, 0, 0, 0
    while spent < max_seconds:
        n = min(n, B - start)
        t0 = time.perf_counter()
        oracle.paged_attention(q[start:start + n], kc, vc, tab[start:start + n],
                               ln[start:start + n], num_kv_heads=step.num_kv_heads,
                               head_dim=step.head_dim, block_size=step.block_size,
                               scale=step.scale, num_blocks=step.num_blocks, threads=threads)
        spent += time.perf_counter() - t0
        done_bytes += int(per_seq_bytes[start:start + n].sum())
        done_seqs += n
        start = (start + n) % B
        per_seq = spent / done_seqs
        n = max(1, min(2 * n, B, int((max_seconds - spent) / per_seq)))
    return dict(value=round(done_bytes / spent / 1e9, 4), unit="GB/s", cores=threads,
                kind="oracle", seconds=round(spent, 3), cpu_model=cpu_model(),
                tokens_per_s=round(done_seqs / spent, 3),
                sample="%d sequence-attentions (%.2f passes over the step's %d sequences), fp64 "
                       "gather + naive softmax attention, %d threads" % (
                           done_seqs, done_seqs / B, B, threads))


TOL = {"fp32": 1e-5, "bf16": 2e-2}


def step_parity(step, pools_before):
    """Every output row of the step against the oracle, and the pools bit
    for bit.  The oracle applies the step's copy-on-write pairs and new
    tokens to the snapshot taken before the first step, then attends over
    every sequence of the batch."""
    import oracle
    import workloads as W
    import torch
    t0 = time.perf_counter()
    kc, vc = pools_before
    hkv, d, bs, N = step.num_kv_heads, step.head_dim, step.block_size, step.num_blocks
    if step.num_pairs:
        oracle.copy_blocks(kc, vc, step.cow_pairs.cpu().numpy(), num_kv_heads=hkv, head_dim=d,
                           block_size=bs, num_blocks=N)
    oracle.reshape_and_cache(W.host_array(step.new_key), W.host_array(step.new_value), kc, vc,
                             step.slot_mapping.cpu().numpy(), num_kv_heads=hkv, head_dim=d,
                             block_size=bs, num_blocks=N)
    pools_ok = (W.host_array(step.key_cache).tobytes() == kc.tobytes() and
                W.host_array(step.value_cache).tobytes() == vc.tobytes())
    ref = oracle.paged_attention(W.host_array(step.query), kc, vc, step.block_tables.cpu().numpy(),
                                 step.context_lens.cpu().numpy(), num_kv_heads=hkv, head_dim=d,
                                 block_size=bs, scale=step.scale, num_blocks=N,
                                 threads=max(1, min(16, os.cpu_count() or 1)))
    got = step.out.double().cpu().numpy()
    dtype = "bf16" if step.query.dtype == torch.bfloat16 else "fp32"
    diff = np.abs(got - ref)
    # A bf16 output is the fp32 result rounded to nearest even: it may also
    # differ by half a bf16 ulp, at most 2^-8 |ref|.
    bound = TOL[dtype] + (2.0 ** -8 * np.abs(ref) if step.out.dtype == torch.bfloat16 else 0.0)
    ok = bool(np.all(diff <= bound)) and bool(np.isfinite(got).all())
    return dict(max_abs_err=float(diff.max()) if diff.size else 0.0, tolerance=TOL[dtype],
                rows=int(got.shape[0] * got.shape[1]), all_rows=True, pools_bit_exact=pools_ok,
                passed=ok and pools_ok, seconds=round(time.perf_counter() - t0, 2))


# ---- bandwidth ceilings -------------------------------------------------------

def load_probe():
    import ctypes
    path = os.path.join(ROOT, "paged_kv_cache_305_amd", "libpaprobe.so")
    if not os.path.exists(path):
        raise SystemExit("libpaprobe.so is missing: build with python -m "
                         "paged_kv_cache_305_amd.build")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.probe_stream_read.argtypes = [vp, i64, vp, i32, i32, i32, vp]
    lib.probe_block_gather.argtypes = [vp, i64, vp, i64, vp, i32, i32, i32, vp]
    lib.probe_stream_read.restype = i32
    lib.probe_block_gather.restype = i32
    return lib


def measure_ceilings(device, flush, reps=5):
    """What the memory system delivers to the decode kernels' access
    patterns on this GPU (libpaprobe.so), best over waves per CU {8, 16},
    blocks in flight {2, 4} and normal / non-temporal loads:
      stream: one 2 GiB buffer read once, in order;
      gather: every 4 KiB block of a 2 GiB pool read once, in random order
              (the paged K/V access pattern);
      cache_gather: a 16 MiB pool read 64 times over in random order, so
              that nearly all reads hit the caches (the shared-prefix
              pattern: a few MB re-read by many waves)."""
    import torch
    lib = load_probe()
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    sink = torch.empty(cus * 16 * 64, dtype=torch.int32, device=device)
    big = 2 << 30
    buf = torch.ones(big // 8, dtype=torch.int64, device=device)
    gen = torch.Generator(device=device).manual_seed(305)
    ids_big = torch.randperm(big // 4096, generator=gen, device=device).to(torch.int32)
    small_blocks = (16 << 20) // 4096
    ids_small = torch.cat([torch.randperm(small_blocks, generator=gen, device=device)
                           for _ in range(64)]).to(torch.int32)

    def timed(launch):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps + 1)]
        for a, b in evs:
            if flush is not None:
                flush.sum()
            a.record()
            rc = launch()
            b.record()
            if rc != 0:
                raise RuntimeError("probe launch failed (%d)" % rc)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs[1:]])) / 1e3

    best = {"stream": (0.0, None), "gather": (0.0, None), "cache_gather": (0.0, None)}
    for wpc in (8, 16):
        for depth in (2, 4):
            for nt in (1, 0):
                shape = dict(waves_per_cu=wpc, depth=depth, nontemporal=bool(nt))
                w = cus * wpc
                t = timed(lambda: lib.probe_stream_read(buf.data_ptr(), big, sink.data_ptr(), w,
                                                        depth, nt, stream))
                if big / t / 1e9 > best["stream"][0]:
                    best["stream"] = (big / t / 1e9, shape)
                t = timed(lambda: lib.probe_block_gather(buf.data_ptr(), big // 4096,
                                                         ids_big.data_ptr(), ids_big.numel(),
                                                         sink.data_ptr(), w, depth, nt, stream))
                if big / t / 1e9 > best["gather"][0]:
                    best["gather"] = (big / t / 1e9, shape)
                n = ids_small.numel()
                t = timed(lambda: lib.probe_block_gather(buf.data_ptr(), small_blocks,
                                                         ids_small.data_ptr(), n,
                                                         sink.data_ptr(), w, depth, nt, stream))
                if n * 4096 / t / 1e9 > best["cache_gather"][0]:
                    best["cache_gather"] = (n * 4096 / t / 1e9, shape)
    del buf, ids_big, ids_small, sink
    torch.cuda.empty_cache()
    out = {k: dict(GBs=round(v[0], 1), frac_of_8TBs=round(v[0] / HBM_PEAK_GBS, 4), best=v[1])
           for k, v in best.items()}
    out["bytes"] = dict(stream=big, gather=big, cache_gather=64 * (16 << 20))
    return out


# ---- one workload -------------------------------------------------------------

def measure_workload(name, args, device, flush, ceilings, parity=True):
    """Time one workload's step (two passes of K steps after W warm-ups) and
    check it against the oracle; returns (result dict, step, lens)."""
    import torch
    import paged_kv_cache_305_amd as pa
    import workloads as W
    log("%s: building the workload" % name)
    step, lens, info = build_step(name, args.partition_size, device,
                                  block_size=args.block_size if name == args.workload else None,
                                  table_order=args.table_order, prefix=not args.no_prefix,
                                  batch=args.batch if name == args.workload else None)
    # The split the library runs for this step (auto: whole segments for short contexts).
    ps = pa.resolve_partition(args.partition_size, step.max_context_len)
    step.fused = {"auto": None, "fused": True, "separate": False}[args.cache_write]
    step.cow_fused = {"auto": None, "fused": True, "separate": False}[args.cow]
    torch.cuda.synchronize()
    pools_before = None
    if parity:
        pools_before = (W.host_array(step.key_cache).copy(), W.host_array(step.value_cache).copy())
    kv_bytes, attn_bytes = algorithmic_bytes(step, lens)
    if step.uses_fused_write:   # the launch also reads and stores each new token's K and V
        attn_bytes += 2 * step.new_key.numel() * step.new_key.element_size() * 2 + \
            step.slot_mapping.numel() * 8
    if step.uses_fused_copy:    # ... and copies each pair's block, K and V (read + write)
        block_bytes = step.num_kv_heads * step.block_size * step.head_dim * \
            step.query.element_size()
        attn_bytes += step.num_pairs * 2 * block_bytes * 2 + step.cow_src.numel() * 8
    K, W_ = args.steps, args.warmup

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()   # torch creates the HIP event on first record; the library re-records it
        return e
    s_ev, e_ev = [ev() for _ in range(K)], [ev() for _ in range(K)]
    ms_ev, me_ev = [ev() for _ in range(K)], [ev() for _ in range(K)]
    gs_ev, ge_ev = [ev() for _ in range(K)], [ev() for _ in range(K)]
    torch.cuda.synchronize()
    for _ in range(W_):
        if flush is not None:
            flush.sum()
        step.run()
    torch.cuda.synchronize()
    # Two passes of K steps.  The first times the step as a caller runs it
    # (value, ms_per_step).  The second has the runtime stamp events with
    # the main kernel's and the merge kernel's own start and end
    # (pa_set_timing_events): their durations.  Events attached to a launch
    # delay the next launch by several microseconds on ROCm, while in a step
    # without events the merge starts as the main kernel ends (kernel
    # traces), so main + merge is the sum of the two durations.
    t0 = time.perf_counter()
    for i in range(K):
        if flush is not None:
            flush.sum()
        s_ev[i].record()
        step.run()
        e_ev[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # A step merges unless every sequence fits one fixed partition.
    merges = ps < 0 or (ps > 0 and step.max_context_len > ps)
    for i in range(K):
        if flush is not None:
            flush.sum()
        pa.set_timing_events(ms_ev[i], me_ev[i], *((gs_ev[i], ge_ev[i]) if merges else ()))
        step.run()
    torch.cuda.synchronize()
    pa.set_timing_events()
    step_ms = [s.elapsed_time(e) for s, e in zip(s_ev, e_ev)]
    main_ms = [s.elapsed_time(e) for s, e in zip(ms_ev, me_ev)]
    merge_ms = [s.elapsed_time(e) for s, e in zip(gs_ev, ge_ev)] if merges else [0.0] * K
    attn_ms = [a + b for a, b in zip(main_ms, merge_ms)]
    t_step = float(np.mean(step_ms)) / 1e3
    t_main = float(np.mean(main_ms)) / 1e3
    t_attn = float(np.mean(attn_ms)) / 1e3
    log("%s: step %.1f us (median %.1f), main kernel %.1f us, main + merge %.1f us" % (
        name, t_step * 1e6, float(np.median(step_ms)) * 1e3, t_main * 1e6, t_attn * 1e6))

    B = int(step.query.shape[0])
    gbs = kv_bytes / t_step / 1e9
    achieved = attn_bytes / t_main / 1e9
    body = "MfmaBody" if (step.query.dtype == torch.bfloat16 and
                          step.query.shape[1] // step.num_kv_heads >= 2) else "ValuBody"
    kernel = "%s<%s>" % ("decode_prefix_tails" if step.prefix_len else
                         "decode_balanced" if ps < 0 else "decode_fixed", body)
    default_variant = (name != args.workload or (
        args.block_size in (None, W.CONFIGS.get(name, {}).get("block_size")) and
        args.batch is None and args.table_order == "random")) and \
        args.cache_write == "auto" and args.cow == "auto" and not args.no_prefix and \
        not args.xcd_weights
    gather = ceilings["gather"]["GBs"] if ceilings else None
    roof = dict(bound="hbm", kernel=kernel, achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                # The committed counters were taken on the workload as it
                # stands (its own block size, batch and placement, default
                # cache write and prefix use): any other variant gets none.
                traffic=counter_traffic(name, ps) if default_variant else None,
                algorithmic_bytes_per_launch=attn_bytes, avg_launch_us=round(t_main * 1e6, 2),
                measured_ceiling_GBs=gather,
                frac_of_measured_ceiling=round(achieved / gather, 4) if gather else None,
                merge_us=round(float(np.mean(merge_ms)) * 1e3, 2),
                main_plus_merge_us=round(t_attn * 1e6, 2),
                main_plus_merge_frac=round(attn_bytes / t_attn / 1e9 / HBM_PEAK_GBS, 4),
                kernel_source_digest=kernel_source_digest())
    result = {
        "metric": "paged decode attention KV GB/s (fraction of HBM peak) and tokens/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "ms_per_step": round(t_step * 1e3, 4),
        "dtype": {torch.bfloat16: "bf16", torch.float32: "fp32"}[step.query.dtype],
        "config": {"workload": WORKLOADS[name] + (
                       " (batch set to %d)" % B if args.batch and name == args.workload else ""),
                   "partition_size": args.partition_size, "partition_resolved": ps,
                   "batch": B, "kv_tokens": int(lens.sum()), "kv_bytes": kv_bytes,
                   "kv_loads": "cached (blocks reused)" if step.kv_reused else "streamed",
                   "shared_prefix_tokens": step.prefix_len,
                   "cache_write": "inside the attention launch" if step.uses_fused_write
                                  else "reshape_and_cache before the attention",
                   "copy_on_write": "none" if not step.num_pairs else
                                    "inside the attention launch" if step.uses_fused_copy
                                    else "copy_blocks before the attention",
                   "flush_between_steps": flush is not None, **info,
                   **block_waste(step, lens)},
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(B / t_step, 1),
        "kv_tokens_per_s": round(float(lens.sum()) / t_step, 1),
        # This step (cache write + attention) repeated for every layer of a
        # model of this shape (32 layers for the 7B shape, 80 for the 70B
        # shape), nothing else of the model: B / (t_step * layers).
        **({"attn_only_model_tokens_per_s": round(B / (t_step * MODEL_LAYERS[name]), 1)}
           if name in MODEL_LAYERS else {}),
        "step_ms_median": round(float(np.median(step_ms)), 4),
        "step_ms_min": round(float(np.min(step_ms)), 4),
        "wall_s_timed_loop": round(wall, 4),
        "roofline": roof,
    }
    if step.prefix_len and ceilings:
        # The shared prompt's tiles are read once per block of 32 query rows
        # (2 MFMA row tiles) of each KV head: cache-level reads of a few MB.
        G = step.query.shape[1] // step.num_kv_heads
        row_blocks = -(-(B * G) // 32)
        per_token = step.num_kv_heads * step.head_dim * 2 * step.query.element_size()
        pf_unique = step.prefix_len * per_token
        cache_bytes = pf_unique * row_blocks
        cg = ceilings["cache_gather"]["GBs"]
        # The prefix's cache-level reads and the tails' HBM reads overlap
        # in one launch: the launch takes at least the longer of the two
        # at the measured ceilings.
        t_hbm = (attn_bytes - pf_unique) / (gather * 1e9)
        t_cache = cache_bytes / (cg * 1e9)
        result["roofline_cache"] = dict(
            bound="cache", kernel=kernel, prefix_unique_bytes=pf_unique,
            prefix_reads_per_tile=row_blocks, cache_bytes_per_launch=cache_bytes,
            achieved=round(cache_bytes / t_main / 1e9, 1), peak=cg, unit="GB/s",
            peak_source="measured cache-level 4 KiB gather (libpaprobe.so)",
            frac=round(cache_bytes / t_main / 1e9 / cg, 4),
            bound_us=round(max(t_hbm, t_cache) * 1e6, 2),
            frac_of_bound=round(max(t_hbm, t_cache) / t_main, 4))
    if args.graph:
        step.capture()
        g_s, g_e = [ev() for _ in range(K)], [ev() for _ in range(K)]
        torch.cuda.synchronize()
        for _ in range(W_):
            if flush is not None:
                flush.sum()
            step.replay()
        for i in range(K):
            if flush is not None:
                flush.sum()
            g_s[i].record()
            step.replay()
            g_e[i].record()
        torch.cuda.synchronize()
        g_ms = [a.elapsed_time(b) for a, b in zip(g_s, g_e)]
        result["graph"] = {"ms_per_step": round(float(np.mean(g_ms)), 4),
                           "step_ms_median": round(float(np.median(g_ms)), 4),
                           "value_GBs": round(kv_bytes / (float(np.mean(g_ms)) / 1e3) / 1e9, 1)}
        log("%s: graph replay: step %.1f us" % (name, float(np.mean(g_ms)) * 1e3))
    if parity:
        result["parity"] = step_parity(step, pools_before)
        log("%s: parity %s, max abs err %.3g over %d rows, pools bit-exact %s" % (
            name, "ok" if result["parity"]["passed"] else "FAILED",
            result["parity"]["max_abs_err"], result["parity"]["rows"],
            result["parity"]["pools_bit_exact"]))
    return result, step, lens


def swap_bench(args, device):
    """Time swap_blocks of every block the 7B-shaped step uses, out to a
    pinned host pool and back in, each direction on its own."""
    import torch
    import paged_kv_cache_305_amd as pa
    import workloads as W
    case = W.make_case("7b", device=device)
    used = np.unique(np.concatenate([case.block_tables[i, :-(-int(L) // case.block_size)]
                                     for i, L in enumerate(case.context_lens)]))
    n = int(used.shape[0])
    hk = torch.empty((n,) + tuple(case.key_cache.shape[1:]), dtype=case.key_cache.dtype,
                     pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    out_map = torch.from_numpy(np.stack([used, np.arange(n)], 1).astype(np.int64)).to(device)
    in_map = torch.from_numpy(np.stack([np.arange(n), used], 1).astype(np.int64)).to(device)
    kw = dict(num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
              block_size=case.block_size)
    nbytes = 2 * n * case.key_cache[0].numel() * case.key_cache.element_size()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) / 1e3

    t_out = timed(lambda: pa.swap_blocks(hk, hv, case.key_cache, case.value_cache, out_map,
                                         **kw))
    t_in = timed(lambda: pa.swap_blocks(case.key_cache, case.value_cache, hk, hv, in_map, **kw))
    ok = W.host_array(hk[:4]).tobytes() == W.host_array(case.key_cache[used[:4]]).tobytes()
    out_gbs, in_gbs = nbytes / t_out / 1e9, nbytes / t_in / 1e9
    result = {
        "metric": "preemption swap GB/s (GPU pool <-> pinned host pool)",
        "value": round((out_gbs + in_gbs) / 2, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t_out + t_in) * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (the 7B-shaped step's K/V pools)",
        "config": {"workload": WORKLOADS["swap"], "blocks": n, "bytes_each_way": nbytes,
                   "swap_out_GBs": round(out_gbs, 2), "swap_in_GBs": round(in_gbs, 2),
                   "copy_checked": ok},
        "roofline": dict(bound="host link", achieved=round((out_gbs + in_gbs) / 2, 2),
                         peak=HOST_LINK_PEAK_GBS, unit="GB/s",
                         frac=round((out_gbs + in_gbs) / 2 / HOST_LINK_PEAK_GBS, 4),
                         traffic=None),
    }
    print(json.dumps(result), flush=True)


def cache_ops_bench(args, device, flush):
    """reshape_and_cache and copy_blocks launched on their own, each timed
    over K launches after W warm-ups (caches flushed before each), and
    checked bit for bit against the oracle's scatter and copy on the whole
    pools.  Algorithmic bytes: the payload read once and written once (plus
    the slots or pairs)."""
    import torch
    import oracle
    import paged_kv_cache_305_amd as pa
    import workloads as W
    from paged_kv_cache_305_amd.step import shared_prefix_step

    def timed(fn):
        for _ in range(args.warmup):
            if flush is not None:
                flush.sum()
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            if flush is not None:
                flush.sum()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) / 1e3

    def entry(kernel, t, alg, payload, ok, **extra):
        return dict(kernel=kernel, avg_launch_us=round(t * 1e6, 2), payload_bytes=payload,
                    algorithmic_bytes_per_launch=alg,
                    roofline=dict(bound="hbm", achieved=round(alg / t / 1e9, 1),
                                  peak=HBM_PEAK_GBS, unit="GB/s",
                                  frac=round(alg / t / 1e9 / HBM_PEAK_GBS, 4)),
                    pools_bit_exact=ok, **extra)

    out = {}
    for name in ("7b", "70b"):
        case = W.make_case(name, device=device)
        kc0, vc0 = W.host_array(case.key_cache).copy(), W.host_array(case.value_cache).copy()
        slots = torch.as_tensor(case.slot_mapping).to(device)
        fn = lambda: pa.reshape_and_cache(case.new_key, case.new_value, case.key_cache,
                                          case.value_cache, slots, block_size=case.block_size,
                                          num_blocks=case.num_blocks)
        t = timed(fn)
        oracle.reshape_and_cache(W.host_array(case.new_key), W.host_array(case.new_value), kc0,
                                 vc0, case.slot_mapping, num_kv_heads=case.num_kv_heads,
                                 head_dim=case.head_dim, block_size=case.block_size,
                                 num_blocks=case.num_blocks)
        ok = (W.host_array(case.key_cache).tobytes() == kc0.tobytes() and
              W.host_array(case.value_cache).tobytes() == vc0.tobytes())
        payload = 2 * case.new_key.numel() * case.new_key.element_size()
        out["reshape_and_cache_" + name] = entry(
            "reshape_and_cache_kernel", t, 2 * payload + 8 * case.batch, payload, ok,
            tokens=case.batch, kv_heads=case.num_kv_heads)
        log("reshape_and_cache (%s): %.2f us, pools bit-exact %s" % (name, t * 1e6, ok))
        del case
        torch.cuda.empty_cache()
    plan = W.shared_plan()
    tens = W.shared_tensors(plan, device=device)
    step, rec = shared_prefix_step(plan, tens, partition_size=-1)
    kc0, vc0 = W.host_array(step.key_cache).copy(), W.host_array(step.value_cache).copy()
    fn = lambda: pa.copy_blocks(step.key_cache, step.value_cache, step.cow_pairs,
                                num_kv_heads=step.num_kv_heads, head_dim=step.head_dim,
                                block_size=step.block_size, num_blocks=step.num_blocks)
    t = timed(fn)
    oracle.copy_blocks(kc0, vc0, rec["pairs"], num_kv_heads=step.num_kv_heads,
                       head_dim=step.head_dim, block_size=step.block_size,
                       num_blocks=step.num_blocks)
    ok = (W.host_array(step.key_cache).tobytes() == kc0.tobytes() and
          W.host_array(step.value_cache).tobytes() == vc0.tobytes())
    block = step.num_kv_heads * step.block_size * step.head_dim * step.query.element_size()
    payload = 2 * step.num_pairs * block
    out["copy_blocks_shared"] = entry("copy_blocks_kernel", t, 2 * payload + 16 * step.num_pairs,
                                      payload, ok, pairs=step.num_pairs)
    log("copy_blocks (%d pairs): %.2f us, pools bit-exact %s" % (step.num_pairs, t * 1e6, ok))
    first = out["reshape_and_cache_7b"]
    result = {
        "metric": "cache kernels: GB/s of payload read + written (reshape_and_cache, copy_blocks)",
        "value": first["roofline"]["achieved"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(first["avg_launch_us"] / 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (the workloads' seeded pools, new tokens and copy pairs)",
        "config": {"workload": WORKLOADS["cacheops"]},
        "roofline": dict(first["roofline"], traffic=None), "kernels": out,
        "parity_all_passed": all(v["pools_bit_exact"] for v in out.values()),
    }
    print(json.dumps(result), flush=True)
    if not result["parity_all_passed"]:
        sys.exit(1)


def copy_calibration(device, steps):
    """A plain 1 GiB device copy, for scaling the FETCH/WRITE counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
    b = torch.empty_like(a)
    for i in range(steps):
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy %d/%d done" % (i + 1, steps))
    print(json.dumps({"copy_bytes": n, "launches": steps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="70b", choices=sorted(WORKLOADS),
                    help="the workload of the headline line (default: the 70B-shaped step)")
    ap.add_argument("--extras", default="7b,long,long32,shared,tiny",
                    help="other workloads timed in the same run and reported under "
                         "\"workloads\" (comma-separated, or none)")
    ap.add_argument("--partition-size", type=int, default=-2,
                    help="tokens per split-K partition; 0 = none, -1 = balanced split, "
                         "-2 = auto (none up to 256 tokens of context, else balanced)")
    ap.add_argument("--no-flush", action="store_true", help="keep caches warm between steps")
    ap.add_argument("--batch", type=int, default=None,
                    help="sequences in the headline step (default: the workload's); lengths "
                         "keep the workload's distribution")
    ap.add_argument("--cache-write", choices=["auto", "fused", "separate"], default="auto",
                    help="write the new tokens inside the attention launch (fused), with "
                         "reshape_and_cache before it (separate); auto = fused")
    ap.add_argument("--cow", choices=["auto", "fused", "separate"], default="auto",
                    help="copy-on-write pairs: inside the attention launch with the new tokens "
                         "(fused, when each pair is a new-token block) or with copy_blocks "
                         "first (separate); auto = fused")
    ap.add_argument("--xcd-weights", default=None,
                    help="per-XCD tile shares of the balanced split, 8 comma-separated ints, or "
                         "two (even,odd) repeated over the 8 XCDs (default: the library's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle check of the timed steps")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the bandwidth-ceiling probes")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--block-size", type=int, default=None,
                    help="block size of the headline workload (default: the workload's own)")
    ap.add_argument("--table-order", choices=["random", "identity"], default="random",
                    help="physical blocks in random order (paged) or consecutive (contiguous)")
    ap.add_argument("--no-prefix", action="store_true",
                    help="shared workload: attend each sequence over its whole table instead "
                         "of reading the shared prompt once for all")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph")
    ap.add_argument("--waste-report", action="store_true",
                    help="only print the allocator's KV waste per workload and block size "
                         "(host only)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the bandwidth ceilings (libpaprobe.so)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_305_amd as pa
    if args.waste_report:
        for row in waste_report():
            print(json.dumps(row), flush=True)
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pa.load()
    if args.xcd_weights:
        wts = [int(x) for x in args.xcd_weights.split(",")]
        pa.set_balance_weights(wts * 4 if len(wts) == 2 else wts)
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.copy_calibration:
        copy_calibration(device, max(1, args.steps))
        return
    if args.workload == "swap":
        swap_bench(args, device)
        return

    flush = None if args.no_flush else torch.ones(1 << 27, dtype=torch.int64, device=device)
    if args.workload == "cacheops":
        cache_ops_bench(args, device, flush)
        return
    ceilings = None
    if not args.no_ceiling or args.ceiling:
        log("measuring the bandwidth ceilings")
        ceilings = measure_ceilings(device, flush)
        log("ceilings: stream %.0f GB/s, 4 KiB gather %.0f GB/s, cache-level gather %.0f GB/s" % (
            ceilings["stream"]["GBs"], ceilings["gather"]["GBs"],
            ceilings["cache_gather"]["GBs"]))
        if args.ceiling:
            print(json.dumps({"ceilings": ceilings}), flush=True)
            return

    result, step, lens = measure_workload(args.workload, args, device, flush, ceilings,
                                          parity=not args.no_parity)
    K, W_ = args.steps, args.warmup
    line = {
        "metric": result.pop("metric"), "value": result.pop("value"), "unit": result.pop("unit"),
        "n_gpus": 1, "steps": K, "warmup": W_, "ms_per_step": result.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": result.pop("dtype"),
        "data": "synthetic (seeded N(0,1) K/V/q, seeded lengths and block permutation)",
        **result,
    }
    if ceilings:
        line["ceilings"] = ceilings
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ~%.0f s, then ~%.0f s on one thread" % (
            args.cpu_seconds, args.cpu_seconds / 3))
        line["cpu_baseline"] = cpu_baseline(step, lens, args.cpu_seconds)
        one = cpu_baseline(step, lens, args.cpu_seconds / 3, threads=1)
        line["cpu_baseline"]["single_thread"] = {
            k: one[k] for k in ("value", "unit", "tokens_per_s", "seconds", "sample")}
    del step
    torch.cuda.empty_cache()
    extras = [] if args.extras in ("", "none") else [x for x in args.extras.split(",")
                                                     if x and x != args.workload]
    if extras:
        line["workloads"] = {}
    for name in extras:
        if name not in WORKLOADS or name in ("swap", "cacheops"):
            raise SystemExit("unknown extra workload %r" % name)
        r, st, _ = measure_workload(name, args, device, flush, ceilings,
                                    parity=not args.no_parity)
        r.pop("metric")
        line["workloads"][name] = r
        del st
        torch.cuda.empty_cache()
    failed = [n for n, r in [(args.workload, line)] + list(line.get("workloads", {}).items())
              if "parity" in r and not r["parity"]["passed"]]
    line["parity_all_passed"] = None if args.no_parity else not failed
    print(json.dumps(line), flush=True)
    if failed:
        log("parity FAILED for: %s" % ", ".join(failed))
        sys.exit(1)


if __name__ == "__main__":
    main()
