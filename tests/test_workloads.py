"""The seeded generators: reproducible, shaped as the pages' workloads, and with
block tables that are valid page assignments."""
import numpy as np
import pytest

import workloads


@pytest.mark.parametrize("cfg", [1, 2, 3, 5, 6])
def test_reproducible(cfg):
    a, b = workloads.make(cfg), workloads.make(cfg)
    assert np.array_equal(a.context_lens, b.context_lens)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.q_packed(), b.q_packed())
    ka, _ = a.tokens(1, 0, 5)
    kb, _ = b.tokens(1, 0, 5)
    assert np.array_equal(ka, kb)


def test_shapes_and_ranges():
    w1 = workloads.make(1)
    assert w1.context_lens.tolist() == [17, 64, 100, 250] and w1.num_pages == 64
    w2 = workloads.make(2)
    assert w2.num_seqs == 64 and w2.context_lens.min() >= 512 and w2.context_lens.max() <= 4096
    assert w2.group_size == 4 and w2.page_size == 64
    w3 = workloads.make(3)
    assert w3.num_prefill == 2 and w3.num_seqs == 258
    assert w3.context_lens[:2].tolist() == [8704, 8704] and w3.new_lens[:2].tolist() == [512, 512]
    Ld = w3.context_lens[2:]
    assert Ld.min() >= 16 and Ld.max() <= 16384 and 700 < np.median(Ld) < 1500
    w4 = workloads.make(4)
    assert (w4.context_lens == 131072).all() and w4.num_splits == 64 and w4.page_size == 128
    w5 = workloads.make(5)
    assert w5.kv_dtype == "fp8" and w5.group_size == 8
    assert w5.context_lens.min() >= 2049 and w5.context_lens.max() <= 8192
    w6 = workloads.make(6)
    assert w6.num_seqs == w6.num_prefill == 64 and (w6.new_lens == 4).all()
    assert w6.context_lens.min() >= 512 and w6.context_lens.max() <= 4096 and w6.group_size == 4


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6])
def test_block_tables_are_valid_assignments(cfg):
    wl = workloads.make(cfg)
    bt = wl.block_tables
    P = wl.page_size
    need = -(-wl.context_lens // P)
    for s in range(wl.num_seqs):
        assert (bt[s, :need[s]] >= 0).all() and (bt[s, need[s]:] == -1).all()
    used = bt[bt >= 0]
    assert used.max() < wl.num_pages
    if wl.prefix_len:
        npre = wl.prefix_len // P
        # members of a group share exactly their prefix pages
        for s in range(wl.num_seqs):
            o = wl.group_owner[wl.group_of[s]]
            assert np.array_equal(bt[s, :npre], bt[o, :npre])
        private = np.concatenate([bt[s, npre:need[s]] for s in range(wl.num_seqs)])
        shared = np.unique(bt[:, :npre])
        assert len(np.unique(private)) == len(private)
        assert not np.isin(private, shared).any()
        assert len(shared) == npre * len(wl.group_owner)
    else:
        assert len(np.unique(used)) == len(used)


def test_history_plan_covers_every_token_once():
    wl = workloads.make(5, num_seqs=6, group_size=3, prefix_len=128, len_range=(129, 300))
    seen = {s: 0 for s in range(wl.num_seqs)}
    for rows, ctx, new, k, v in wl.history_plan():
        assert k.shape[0] == int(new.sum()) == v.shape[0]
        for r, c, n in zip(rows, ctx, new):
            if n == wl.prefix_len and c == wl.prefix_len and r in wl.group_owner:
                for s in np.flatnonzero(wl.group_of == wl.group_of[r]):
                    seen[s] += n
            else:
                seen[r] += n
    for s in range(wl.num_seqs):
        assert seen[s] == wl.context_lens[s] - wl.new_lens[s]
