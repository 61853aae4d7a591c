"""Pins of the oracle's paged attention against facts fixed outside it.

* P1  dense attention (torch SDPA, float64) over the workload's *logical* tokens,
      which never pass through a page pool, equals the oracle's paged result;
* P2  permuting physical pages (and the tables with them) leaves it bit-identical;
* P3  softmax weights sum to 1;
* P4  append changes exactly the slots the block tables name;
* P5  closed forms (one key, zero query, equal keys, one dominant key);
* P6  page size = max length with an identity table is the contiguous cache layout;
* P7  any split of the keys merged by log-sum-exp equals the unsplit result;
* P9  the pages' worked block-table example (golden fixture);
* P10 a prompt run as chunks equals one causal prefill;
* P11 decode equals the last row of a one-token chunk and of a full causal prefill.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from tests.oracle_state import oracle_outputs, oracle_pool, scales

HERE = os.path.dirname(os.path.abspath(__file__))

SMALL = {
    1: dict(),
    2: dict(num_seqs=5, len_range=(1, 300)),
    3: dict(num_seqs=6, num_prefill=2, prefill_chunk=70, prefill_cached=130, median=40,
            clip=(1, 200)),
    4: dict(num_seqs=2, context_len=700, num_splits=4),
    5: dict(num_seqs=6, group_size=3, prefix_len=128, len_range=(129, 400)),
}


def logical_f64(wl, arr):
    """Storage values -> float64 through torch's own casts (independent of oracle.to_f64)."""
    if arr.dtype == np.float32:
        return torch.from_numpy(arr).double()
    return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).double()


def logical_kv(wl, s):
    """Sequence s's K/V [L][Hkv][D] as float64 straight from the generator, quantized
    and dequantized with torch's float8_e4m3fn cast for an FP8 cache."""
    k, v = wl.tokens(s)
    k, v = logical_f64(wl, k), logical_f64(wl, v)
    if wl.kv_dtype == "fp8":
        ks, vs, kinv, vinv = wl.fp8_scales()
        out = []
        for x, sc, inv in ((k, ks, kinv), (v, vs, vinv)):
            x32 = x.float() * torch.from_numpy(inv)[None, :, None]
            q8 = x32.to(torch.float8_e4m3fn).double()
            out.append(q8 * torch.from_numpy(sc).double()[None, :, None])
        k, v = out
    if wl.kv_dtype == "mxfp4":   # the codec itself is pinned in test_oracle_mxfp4.py
        k, v = (torch.from_numpy(oracle.mx_decode(*oracle.mx_encode(x.numpy()))) for x in (k, v))
    return k, v


def sdpa_reference(wl):
    """Dense causal attention over logical tokens: decode rows and prefill rows."""
    q = logical_f64(wl, wl.q_packed())
    cu = wl.cu(wl.new_lens)
    G = wl.group_size
    out = torch.zeros_like(q)
    for s in range(wl.num_seqs):
        L, C = int(wl.context_lens[s]), int(wl.new_lens[s])
        k, v = logical_kv(wl, s)
        kr = k.repeat_interleave(G, dim=1).permute(1, 0, 2)[None]     # [1][Hq][L][D]
        vr = v.repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
        qs = q[cu[s]:cu[s + 1]].permute(1, 0, 2)[None]                  # [1][Hq][C][D]
        pos = torch.arange(L - C, L)[:, None]
        mask = torch.arange(L)[None, :] <= pos                          # [C][L]
        o = F.scaled_dot_product_attention(qs, kr, vr, attn_mask=mask,
                                           scale=float(np.float32(wl.sm_scale)))
        out[cu[s]:cu[s + 1]] = o[0].permute(1, 0, 2)
    return out.numpy()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_p1_paged_oracle_equals_dense_attention(cfg):
    wl = workloads.make(cfg, **SMALL[cfg])
    pool = oracle_pool(wl)
    dec, _, pf, _ = oracle_outputs(wl, pool)
    ref = sdpa_reference(wl)
    npf = wl.num_prefill
    cu = wl.cu(wl.new_lens)
    got = np.concatenate([pf, dec]) if npf else dec
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    assert np.isfinite(got).all()


@pytest.mark.parametrize("cfg,over", [
    (2, dict(num_seqs=4, len_range=(1, 300), kv_dtype="mxfp4")),
    (3, dict(num_seqs=5, num_prefill=2, prefill_chunk=[40, 3], prefill_cached=[70, 33], median=40,
             clip=(1, 150), kv_dtype="mxfp4")),
])
def test_p1_mxfp4_pool_equals_dense_attention_over_decoded_tokens(cfg, over):
    """An MXFP4 pool (rows of codes and scales in paged slots) attends exactly like
    dense attention over the decoded logical tokens."""
    wl = workloads.make(cfg, **over)
    pool = oracle_pool(wl)
    dec, _, pf, _ = oracle_outputs(wl, pool)
    ref = sdpa_reference(wl)
    got = np.concatenate([pf, dec]) if wl.num_prefill else dec
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_p1_catches_a_planted_head_mapping_error(monkeypatch):
    """A plausible mistake (query head h reading kv head h % Hkv instead of h // G)
    must fail the dense-attention pin."""
    wl = workloads.make(2, **SMALL[2])
    pool = oracle_pool(wl)
    ref = sdpa_reference(wl)
    real = oracle.paged_attention.gather

    def wrong_gather(pool_, row, L, g, *a, **k):
        return real(pool_, row, L, (g + 1) % wl.num_kv_heads, *a, **k)

    monkeypatch.setattr(oracle.paged_attention, "gather", wrong_gather)
    dec, _, _, _ = oracle_outputs(wl, pool)
    assert np.abs(dec - ref).max() > 1e-3


@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_p2_page_permutation_is_bit_identical(cfg):
    wl = workloads.make(cfg, **SMALL[cfg])
    pool = oracle_pool(wl)
    a = oracle_outputs(wl, pool)
    perm = np.random.default_rng(7).permutation(wl.num_pages)
    pool2 = np.empty_like(pool)
    pool2[perm] = pool                      # page p moves to perm[p]
    bt = wl.block_tables
    wl.block_tables = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    b = oracle_outputs(wl, pool2)
    for x, y in zip(a, b):
        if x is not None:
            assert np.array_equal(x, y)


def test_p3_weights_sum_to_one():
    wl = workloads.make(2, **SMALL[2])
    pool = oracle_pool(wl)
    _, _, w = oracle.decode(pool, wl.block_tables, wl.context_lens, wl.q_packed(), wl.q_dtype,
                            wl.sm_scale, wl.kv_dtype, return_weights=True)
    for (s, g), ws in w.items():
        assert ws.shape == (wl.group_size, wl.context_lens[s])
        np.testing.assert_allclose(ws.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert (ws >= 0).all()


@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_p4_append_writes_exactly_the_named_slots(cfg):
    wl = workloads.make(cfg, **SMALL[cfg])
    before = oracle_pool(wl, include_step=False)
    after = before.copy()
    _, _, kinv, vinv = scales(wl)
    k, v = wl.step_kv()
    W = oracle.append(after, wl.block_tables, wl.context_lens, wl.new_lens, k, v, wl.in_dtype,
                      wl.kv_dtype, kinv, vinv)
    assert len(W) == int(wl.new_lens.sum()) == len(set(W))
    changed = np.zeros(after.shape[:1] + after.shape[3:4], bool)     # [page][slot]
    for p, t in W:
        changed[p, t] = True
    diff = (before.view(np.uint8) != after.view(np.uint8)).reshape(
        after.shape[0], 2, wl.num_kv_heads, wl.page_size, -1).any(axis=(1, 2, 4))
    assert not (diff & ~changed).any(), "append touched a slot no table names"
    # each written slot holds the encoded new rows, independent of the old value
    row = 0
    for s in range(wl.num_seqs):
        L, n = int(wl.context_lens[s]), int(wl.new_lens[s])
        for j in range(n):
            t = L - n + j
            p = wl.block_tables[s][t // wl.page_size]
            want_k = oracle.encode_rows(k[row:row + 1], wl.in_dtype, wl.kv_dtype, kinv)[0]
            assert np.array_equal(after[p, 0, :, t % wl.page_size].view(np.uint8),
                                  want_k.view(np.uint8))
            row += 1
    # and no shared-prefix page is ever a target of the step's append
    if wl.prefix_len:
        shared = set(np.unique(wl.block_tables[:, :wl.prefix_len // wl.page_size]).tolist())
        assert not shared & {p for p, _ in W}


def test_p5_closed_forms():
    rng = np.random.default_rng(3)
    D = 16
    V = rng.standard_normal((9, D))
    K = rng.standard_normal((9, D))
    q = rng.standard_normal((2, D))
    # a single key: the output is that key's value row, exactly
    o, lse = oracle.attend_rows(q, K[:1], V[:1], 0.25)
    assert np.array_equal(o, np.repeat(V[:1], 2, axis=0))
    np.testing.assert_allclose(lse, 0.25 * (q @ K[0]), rtol=0, atol=1e-14)
    # a zero query weighs all keys equally: the mean of V
    o, lse = oracle.attend_rows(np.zeros((1, D)), K, V, 0.25)
    np.testing.assert_allclose(o[0], V.mean(axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(9.0), rtol=0, atol=1e-14)
    # identical keys: the mean of V
    o, _ = oracle.attend_rows(q, np.repeat(K[:1], 9, axis=0), V, 0.25)
    np.testing.assert_allclose(o, np.repeat(V.mean(axis=0)[None], 2, axis=0), atol=1e-14)
    # one logit 200 above the rest: that value row (exactly so in float32)
    Kd = np.zeros((9, D))
    Kd[4, 0] = 200.0
    o, _ = oracle.attend_rows(np.eye(D)[:1], Kd, V, 1.0)
    assert np.array_equal(o.astype(np.float32), V[4:5].astype(np.float32))


def test_p6_identity_table_is_the_contiguous_layout():
    """Page size = max length, sequence s owns page s: the pool is the contiguous
    cache [batch][2][heads][max_seq_len][head_dim]."""
    wl = workloads.make(2, num_seqs=4, len_range=(5, 40))
    maxL = int(wl.context_lens.max())
    P = 64
    assert maxL <= P
    pool = oracle.new_pool(4, wl.num_kv_heads, P, wl.head_dim, "bf16", fill=0)
    bt = np.arange(4, dtype=np.int32)[:, None]
    ks, vs = zip(*[wl.tokens(s) for s in range(4)])
    oracle.append(pool, bt, wl.context_lens, wl.context_lens, np.concatenate(ks),
                  np.concatenate(vs), "bf16", "bf16")
    contig = np.zeros_like(pool)
    for s in range(4):
        L = int(wl.context_lens[s])
        contig[s, 0, :, :L] = ks[s].transpose(1, 0, 2)
        contig[s, 1, :, :L] = vs[s].transpose(1, 0, 2)
    assert np.array_equal(pool, contig)


def test_p7_partition_merge_equals_unsplit():
    rng = np.random.default_rng(11)
    L, D = 1000, 32
    K, V = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    q = rng.standard_normal((4, D)) * 3
    ref, ref_lse = oracle.attend_rows(q, K, V, 0.2)
    for cuts in ([0, L], [0, 128, 256, 999, L], [0, 0, 500, 500, L],
                 sorted(rng.integers(0, L, 20).tolist() + [0, L])):
        parts = [oracle.partition_stats(q, K, V, 0.2, a, b) for a, b in zip(cuts, cuts[1:])]
        o, lse = oracle.lse_merge(parts)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_p9_pages_worked_block_table_example():
    g = json.load(open(os.path.join(HERE, "golden", "block_table_example.json")))
    row = np.array(g["block_table"], np.int32)
    for t, page, slot in g["cases"]:
        assert oracle.slot_of(row, t, g["page_size"]) == (page, slot)


def _prompt_pool(wl, T, P=16):
    """A pool holding nothing yet, one sequence of T tokens whose pages are 5,2,9,..."""
    npages = -(-T // P)
    bt = np.array([(7 * i + 5) % (npages + 3) for i in range(npages)], np.int32)[None]
    pool = oracle.new_pool(npages + 3, wl.num_kv_heads, P, wl.head_dim, "bf16", fill=0)
    return pool, bt


def test_p10_chunked_prefill_equals_one_causal_prefill():
    wl = workloads.make(2, num_seqs=1, len_range=(150, 150))
    T = 150
    k, v = wl.tokens(0)
    q = workloads.to_storage(np.random.default_rng(5).standard_normal(
        (T, wl.num_q_heads, wl.head_dim)).astype(np.float32), "bf16")
    pool, bt = _prompt_pool(wl, T)
    oracle.append(pool, bt, [T], [T], k, v, "bf16", "bf16")
    full, full_lse = oracle.prefill_chunk(pool, bt, [T], [0, T], q, "bf16", wl.sm_scale, "bf16")
    pool2, _ = _prompt_pool(wl, T)
    outs, lses = [], []
    cuts = [0, 32, 64, 128, 150]          # chunks are multiples of the page size but the last
    for a, b in zip(cuts, cuts[1:]):
        oracle.append(pool2, bt, [b], [b - a], k[a:b], v[a:b], "bf16", "bf16")
        o, l = oracle.prefill_chunk(pool2, bt, [b], [0, b - a], q[a:b], "bf16", wl.sm_scale, "bf16")
        outs.append(o)
        lses.append(l)
    np.testing.assert_allclose(np.concatenate(outs), full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(lses), full_lse, rtol=0, atol=1e-12)


def test_p11_decode_is_the_last_row_of_a_causal_prefill():
    wl = workloads.make(2, num_seqs=1, len_range=(97, 97))
    T = 97
    k, v = wl.tokens(0)
    q = workloads.to_storage(np.random.default_rng(6).standard_normal(
        (T, wl.num_q_heads, wl.head_dim)).astype(np.float32), "bf16")
    pool, bt = _prompt_pool(wl, T)
    oracle.append(pool, bt, [T], [T], k, v, "bf16", "bf16")
    full, _ = oracle.prefill_chunk(pool, bt, [T], [0, T], q, "bf16", wl.sm_scale, "bf16")
    one, _ = oracle.prefill_chunk(pool, bt, [T], [0, 1], q[-1:], "bf16", wl.sm_scale, "bf16")
    dec, _ = oracle.decode(pool, bt, [T], q[-1:], "bf16", wl.sm_scale, "bf16")
    np.testing.assert_allclose(dec[0], one[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dec[0], full[-1], rtol=0, atol=1e-12)


def test_bf16_widening_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ours = oracle.paged_attention.to_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
