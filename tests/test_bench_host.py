"""Host arithmetic of bench.py (no GPU): the prefill call's exact causal flops, the
unique bytes of a shared-prefix batch and the paged-vs-static memory report."""
import numpy as np

import bench
import workloads


def test_prefill_flops_of_the_mixed_batch():
    # 2 requests x 32 query heads x sum over 512 queries of (8193 + i) keys x 128 dims x 4
    wl = workloads.make(3)
    expect = 2 * 32 * sum(8193 + i for i in range(512)) * 128 * 4
    assert bench.prefill_flops(wl) == expect
    assert abs(expect - 141.7e9) < 0.1e9


def test_prefill_flops_under_a_window_count_only_visible_keys():
    wl = workloads.make(3, num_seqs=3, num_prefill=1, prefill_chunk=10, prefill_cached=50, window=8)
    # every query sees exactly 8 keys (its own and the 7 before it)
    assert bench.prefill_flops(wl) == 10 * 8 * 4 * wl.head_dim * wl.num_q_heads


def test_unique_tokens_count_a_shared_prefix_once():
    wl = workloads.make(5, num_seqs=8, group_size=4, prefix_len=128, len_range=(129, 400))
    rows = range(wl.num_seqs)
    total = int(wl.context_lens.sum())
    groups = wl.num_seqs // 4
    assert bench.unique_kv_tokens(wl, rows) == total - (4 - 1) * 128 * groups
    wl2 = workloads.make(2, num_seqs=6, len_range=(1, 300))
    assert bench.unique_kv_tokens(wl2, range(6)) == int(wl2.context_lens.sum())


def test_memory_report_against_static_reservation():
    wl = workloads.make(1)        # lengths 17, 64, 100, 250 on pages of 16
    m = bench.memory_report(wl)
    assert m["pages_paged"] == 2 + 4 + 7 + 16
    assert m["pages_static_reservation"] == 4 * 16
    assert np.isclose(m["saving"], 1 - 29 / 64, atol=1e-4)
