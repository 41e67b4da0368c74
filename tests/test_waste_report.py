"""The block-size waste report (bench.py --waste-report) against closed
forms: for independent sequences the allocator's waste is
sum(ceil(L/Bs)*Bs - L) / sum(ceil(L/Bs)*Bs), under one block per sequence
(note-023 Key results and Concepts), and paging needs less memory than
reserving the maximum context per sequence."""
import numpy as np

import bench
import workloads as W


def test_waste_report_matches_closed_forms():
    rows = bench.waste_report(block_sizes=(8, 16, 64))
    assert len(rows) == 4 * 3
    for r in rows:
        bs = r["block_size"]
        if r["workload"] != "shared":
            L = np.asarray(W.case_structure(r["workload"], block_size=bs).lengths, np.int64)
            alloc = int(np.sum(-(-L // bs) * bs))
            assert r["slots_allocated"] == alloc
            assert r["paged_waste"] == round(1 - L.sum() / alloc, 5)
            assert alloc - L.sum() < bs * len(L)
            assert r["contiguous_waste"] == round(1 - L.sum() / (len(L) *
                                                                 bench.MAX_CONTEXT[r["workload"]]), 5)
        assert r["paged_over_contiguous_memory"] <= 1.0
    shared16 = [r for r in rows if r["workload"] == "shared" and r["block_size"] == 16][0]
    # The prompt is stored once for 64 sequences: far less memory than 64 copies.
    assert shared16["paged_over_contiguous_memory"] < 0.1
