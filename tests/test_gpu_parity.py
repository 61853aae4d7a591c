"""GPU parity of the HIP path against the CPU fp64 oracle, through the C ABI.

Small variants of the five workloads (several pages and partitions, ragged tails)
are compared element by element; kv_append and page gather are compared bit for
bit.  Full-size workloads are in test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_common import assert_close, assert_lse_close, pool_from_token_major, pool_token_major
from tests.oracle_state import oracle_outputs, oracle_pool

pytestmark = pytest.mark.gpu

SMALL = {
    "cfg1": (1, dict()),
    "cfg2s": (2, dict(num_seqs=7, len_range=(1, 700))),
    "cfg3s": (3, dict(num_seqs=9, num_prefill=2, prefill_chunk=70, prefill_cached=190, median=60,
                      clip=(1, 400))),
    "cfg4s": (4, dict(num_seqs=2, context_len=1500, num_splits=5)),
    "cfg5s": (5, dict(num_seqs=6, group_size=3, prefix_len=128, len_range=(129, 600))),
}


def _batch(gpu_lib, name, num_splits=None, **extra):
    from tests.device_batch import DeviceBatch
    cfg, over = SMALL[name]
    wl = workloads.make(cfg, **{**over, **extra})
    print(f"[case] {name} S={wl.num_seqs} Lmax={wl.max_context_len} kv={wl.kv_dtype}", flush=True)
    db = DeviceBatch(wl, num_splits=num_splits)
    db.fill_history()
    db.prepare_step()
    return wl, db


@pytest.mark.parametrize("name", list(SMALL))
def test_append_is_bit_exact(gpu_lib, name):
    wl, db = _batch(gpu_lib, name)
    db.append_step()
    torch.cuda.synchronize()
    ref = oracle_pool(wl)
    got = pool_token_major(db.pool_bits())
    assert got.shape == ref.shape
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), \
        f"{int((got.view(np.uint8) != ref.view(np.uint8)).sum())} bytes differ"


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_routes_rows_across_many_sequences(gpu_lib, kv):
    """kv_append over 300 sequences (more than one workgroup samples at once, so the row
    owner is found in two rounds) where only every third sequence has a new row: each
    row lands in its own sequence's slot and sequences without rows keep their bytes."""
    from paged_kv_cache_413_amd import binding as B
    from tests.device_batch import DeviceBatch, to_device
    wl = workloads.make(2, num_seqs=300, len_range=(2, 90), kv_dtype=kv)
    print(f"[case] sparse append S={wl.num_seqs} kv={kv}", flush=True)
    db = DeviceBatch(wl)
    db.fill_history()
    new = (np.arange(wl.num_seqs) % 3 == 1).astype(np.int32)
    k, v = wl.step_kv()  # one row per sequence; keep those of the sequences that append
    k, v = k[new == 1], v[new == 1]
    seqs = B.make_seqs(db.block_tables, db.context_lens, wl.max_context_len)
    cu = torch.from_numpy(wl.cu(new)).to(db.dev)
    B.kv_append(db.cache, seqs, to_device(k, wl.in_dtype, db.dev), to_device(v, wl.in_dtype, db.dev),
                cu, int(new.sum()))
    torch.cuda.synchronize()
    ref = oracle_pool(wl, include_step=False)
    kinv, vinv = wl.fp8_scales()[2:] if kv == "fp8" else (None, None)
    oracle.append(ref, wl.block_tables, wl.context_lens, new, k, v, wl.in_dtype, wl.kv_dtype, kinv, vinv)
    got = pool_token_major(db.pool_bits())
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), \
        f"{int((got.view(np.uint8) != ref.view(np.uint8)).sum())} bytes differ"


@pytest.mark.parametrize("name", list(SMALL))
def test_debug_gather_is_bit_exact(gpu_lib, name):
    from paged_kv_cache_413_amd import binding as B
    wl, db = _batch(gpu_lib, name)
    db.append_step()
    S, Lm, H, D = wl.num_seqs, wl.max_context_len, wl.num_kv_heads, wl.head_dim
    kout = torch.zeros((S, Lm, H, D), dtype=db.pool.dtype, device=db.dev)
    vout = torch.zeros_like(kout)
    B.paged_kv_debug_gather(db.cache, db.seqs_all, kout, vout)
    torch.cuda.synchronize()
    view = {"f32": torch.int32, "bf16": torch.int16, "fp8": torch.uint8}[wl.kv_dtype]
    kg, vg = kout.view(view).cpu().numpy(), vout.view(view).cpu().numpy()
    pool = oracle_pool(wl) if wl.kv_dtype == "fp8" else None
    for s in range(S):
        L = int(wl.context_lens[s])
        if wl.kv_dtype == "fp8":
            ks, vs, _, _ = wl.fp8_scales()
            for g in range(H):
                K, V = oracle.gather(pool, wl.block_tables[s], L, g, "fp8", ks, vs)
                assert np.array_equal(oracle.decode_e4m3(kg[s, :L, g]) * np.float64(ks[g]), K)
                assert np.array_equal(oracle.decode_e4m3(vg[s, :L, g]) * np.float64(vs[g]), V)
        else:
            k, v = wl.tokens(s)
            assert np.array_equal(kg[s, :L].view(k.dtype), k)
            assert np.array_equal(vg[s, :L].view(v.dtype), v)
        assert (kg[s, L:] == 0).all() and (vg[s, L:] == 0).all()


@pytest.mark.parametrize("name", list(SMALL))
def test_attention_matches_oracle(gpu_lib, name):
    wl, db = _batch(gpu_lib, name)
    db.step()
    torch.cuda.synchronize()
    dec, dec_lse, pf, pf_lse = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    err = assert_close(dec, ref[0], wl.kv_dtype, "decode")
    assert_lse_close(dec_lse, ref[1], wl.kv_dtype, "decode")
    if wl.num_prefill:
        assert_close(pf, ref[2], wl.kv_dtype, "prefill")
        assert_lse_close(pf_lse, ref[3], wl.kv_dtype, "prefill")
    print(f"[ok] {name} decode err {err:.3e}", flush=True)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_split_count_only_moves_rounding(gpu_lib, splits):
    wl, db = _batch(gpu_lib, "cfg4s", num_splits=splits)
    db.step()
    torch.cuda.synchronize()
    dec, lse, _, _ = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    assert_close(dec, ref[0], "bf16", f"splits={splits}")
    assert_lse_close(lse, ref[1], "bf16", f"splits={splits}")


@pytest.mark.parametrize("name", ["cfg1", "cfg3s", "cfg5s"])
def test_page_permutation_is_bit_identical(gpu_lib, name):
    """Outputs depend on logical positions only: moving every page to another physical
    id (and rewriting the tables to match) changes no bit of the result."""
    wl, db = _batch(gpu_lib, name)
    db.step()
    torch.cuda.synchronize()
    a = [t.clone() for t in (db.out_dec, db.lse_dec)] + \
        ([db.out_pf.clone(), db.lse_pf.clone()] if wl.num_prefill else [])
    perm = np.random.default_rng(1).permutation(wl.num_pages)
    bt = wl.block_tables
    wl2 = workloads.make(SMALL[name][0], **SMALL[name][1])
    wl2.block_tables = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    from tests.device_batch import DeviceBatch
    db2 = DeviceBatch(wl2)
    db2.fill_history()
    db2.step()
    torch.cuda.synchronize()
    b = [db2.out_dec, db2.lse_dec] + ([db2.out_pf, db2.lse_pf] if wl.num_prefill else [])
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.uint8) if y.dtype != torch.float32 else y.view(torch.int32))


def test_edge_lengths_and_tiny_pages(gpu_lib):
    """Lengths 1, P-1, P, P+1 and a 2-token page size."""
    from tests.device_batch import DeviceBatch
    for P, lens in ((2, [1, 2, 3, 5, 64]), (16, [1, 15, 16, 17, 33]), (64, [1, 63, 64, 65, 300])):
        wl = workloads.make(1, lens=lens, page_size=P, num_pages=-(-max(lens) // P) * len(lens) + 3)
        print(f"[case] edge P={P} lens={lens}", flush=True)
        db = DeviceBatch(wl)
        db.fill_history()
        db.step()
        torch.cuda.synchronize()
        dec, lse, _, _ = db.outputs_f64()
        ref = oracle_outputs(wl, oracle_pool(wl))
        assert_close(dec, ref[0], "f32", f"P={P}")
        assert_lse_close(lse, ref[1], "f32", f"P={P}")
        # length 1: the output is the appended V row itself
        assert np.allclose(dec[0], wl.tokens(0)[1][0].repeat(wl.group_size, axis=0), atol=1e-6)


def test_one_hot_probe_checks_gather_through_attention(gpu_lib):
    """A query aligned with one key that is far larger than the rest returns exactly
    that key's V row: the attention kernel read the right slot of the right page."""
    from tests.device_batch import DeviceBatch
    wl = workloads.make(2, num_seqs=3, len_range=(200, 500))
    db = DeviceBatch(wl)
    db.fill_history()
    db.prepare_step()
    db.append_step()
    torch.cuda.synchronize()
    # overwrite K of one chosen token per sequence, on a token-major host copy
    pool = pool_token_major(db.pool_bits()).view(np.uint16).copy()   # bf16 bits
    big = np.array([64.0], np.float32).view(np.uint32)[0] >> 16
    target = [7, 130, int(wl.context_lens[2]) - 1]
    for s, t in enumerate(target):
        page, slot = int(wl.block_tables[s][t // wl.page_size]), t % wl.page_size
        pool[page, 0, :, slot, :] = 0
        pool[page, 0, :, slot, 0] = big
    stored = pool_from_token_major(pool)
    db.pool.copy_(torch.from_numpy(stored.view(np.int16)).view(torch.bfloat16).to(db.dev))
    q = torch.zeros_like(db.q_dec)
    q[:, :, 0] = 64.0
    db.q_dec.copy_(q)
    db.decode_step()
    torch.cuda.synchronize()
    out = db.out_dec.float().cpu()
    for s, t in enumerate(target):
        page, slot = int(wl.block_tables[s][t // wl.page_size]), t % wl.page_size
        v = torch.from_numpy(pool[page, 1, :, slot, :].astype(np.int16)).view(torch.bfloat16).float()
        want = v.repeat_interleave(wl.group_size, dim=0)
        assert torch.equal(out[s], want), s


MFMA_EDGES = [
    # (page_size, lens, num_q_heads, num_kv_heads, head_dim, num_splits)
    (8, [1, 7, 8, 9, 31, 32, 33, 100], 32, 8, 128, 0),
    (16, [1, 15, 16, 17, 63, 64, 65, 200], 8, 8, 64, 0),
    (32, [1, 31, 32, 33, 95, 300], 16, 8, 128, 0),
    (64, [1, 2, 63, 64, 65, 129, 1000], 64, 8, 128, 0),
    (128, [1, 127, 128, 129, 700], 32, 2, 64, 0),
    (64, [1, 63, 64, 65, 700, 2100], 32, 8, 128, 3),
    (16, [5, 40, 333], 16, 1, 128, 4),
]


@pytest.mark.parametrize("P,lens,hq,hkv,D,ns", MFMA_EDGES)
def test_mfma_decode_edge_shapes(gpu_lib, P, lens, hq, hkv, D, ns):
    """The matrix-core decode kernels on ragged lengths around page and 32-token
    block edges, pages of 8..128 tokens, groups of 1..16 query heads per kv head,
    head_dim 64 and 128, balanced and fixed partitions."""
    from tests.device_batch import DeviceBatch
    wl = workloads.make(2, lens=lens, page_size=P, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
                        num_splits=ns)
    print(f"[case] mfma edge P={P} lens={lens} Hq={hq} Hkv={hkv} D={D} splits={ns}", flush=True)
    db = DeviceBatch(wl)
    db.fill_history()
    db.step()
    torch.cuda.synchronize()
    dec, lse, _, _ = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    assert_close(dec, ref[0], "bf16", f"P={P}")
    assert_lse_close(lse, ref[1], "bf16", f"P={P}")


@pytest.mark.parametrize("kv,num_seqs,splits", [("bf16", 3000, 0), ("bf16", 3000, 2), ("fp8", 1000, 0),
                                                 ("bf16", 257, 0)])
def test_many_short_sequences(gpu_lib, kv, num_seqs, splits):
    """Hundreds to thousands of decode sequences of 1..80 tokens (Llama-3-8B heads, pages
    of 64; 257 is one past the sequences each balanced-kernel wave caches in registers):
    the balanced schedule's search over sequences runs many 64-sequence rounds and its
    shares hold many whole segments; fixed partitions give most sequences one."""
    from tests.device_batch import DeviceBatch
    wl = workloads.make(2, num_seqs=num_seqs, len_range=(1, 80), kv_dtype=kv, num_splits=splits)
    print(f"[case] many sequences S={num_seqs} kv={kv} splits={splits}", flush=True)
    db = DeviceBatch(wl)
    db.fill_history()
    db.step()
    torch.cuda.synchronize()
    dec, lse, _, _ = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    assert_close(dec, ref[0], kv, f"S={num_seqs}")
    assert_lse_close(lse, ref[1], kv, f"S={num_seqs}")


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_dense_fp8_decode_past_one_wave_per_segment(gpu_lib, kv):
    """One-query FP8 calls with more (sequence, kv head) segments than one wave per SIMD
    gives waves run the dense kernel (raw FP8 blocks, two waves per SIMD: twice the waves,
    so a larger workspace); fewer segments, or bf16 caches, keep the one-wave kernel.
    Both match the oracle."""
    from tests.device_batch import DeviceBatch
    sizes = {}
    for S in (100, 200):                       # 800 and 1 600 segments of 8 kv heads
        wl = workloads.make(2, num_seqs=S, len_range=(1, 200), kv_dtype=kv, num_splits=0)
        print(f"[case] dense decode kv={kv} S={S}", flush=True)
        db = DeviceBatch(wl)
        db.fill_history()
        db.step()
        torch.cuda.synchronize()
        dec, lse, _, _ = db.outputs_f64()
        ref = oracle_outputs(wl, oracle_pool(wl))
        assert_close(dec, ref[0], kv, f"S={S}")
        assert_lse_close(lse, ref[1], kv, f"S={S}")
        sizes[S] = db.ws_dec_bytes
    if kv == "fp8":
        assert sizes[200] > 1.5 * sizes[100], sizes     # twice the waves, twice the records
    else:
        assert sizes[200] == sizes[100], sizes          # same resident waves either way


AUTO_WAVES = [
    # (waves, workload, overrides): few waves, so shares are long and spread over
    # several (sequence, kv head) segments, and segments over several waves
    (3, 2, dict(lens=[1, 63, 700, 2100, 33], page_size=64, num_q_heads=32, num_kv_heads=8,
                head_dim=128)),
    (16, 2, dict(lens=[1, 63, 700, 2100, 33], page_size=32, num_q_heads=8, num_kv_heads=8,
                 head_dim=64)),                                    # G = 1
    (12, 2, dict(lens=[5, 40, 333, 1000, 17, 64], page_size=16, num_q_heads=16, num_kv_heads=2,
                 head_dim=64)),                                    # G = 8, pages of 16
    (40, 2, dict(lens=[1, 31, 32, 33, 95, 300, 4000], page_size=8, num_q_heads=128,
                 num_kv_heads=8, head_dim=128)),                   # G = 16, pages of 8
    (20, 5, dict(num_seqs=6, group_size=3, prefix_len=128, len_range=(129, 600))),  # fp8 KV, 48 segments: dense
    (30, 5, dict(num_seqs=3, group_size=3, prefix_len=128, len_range=(129, 900))),  # fp8 KV, 24 segments: one wave/SIMD
    (12, 2, dict(lens=[1, 63, 700, 2100, 33, 300], page_size=128, num_q_heads=16, num_kv_heads=4,
                 head_dim=64, kv_dtype="fp8")),                    # fp8, D = 64, pages of 128: dense
    (8, 2, dict(lens=[1, 95, 700, 1500, 33], page_size=64, num_q_heads=128, num_kv_heads=8,
                head_dim=128, kv_dtype="fp8")),                    # fp8 dense, G = 16
    (6, 2, dict(lens=[31, 64, 650, 1200, 2], page_size=32, num_q_heads=8, num_kv_heads=8,
                head_dim=64, kv_dtype="fp8")),                     # fp8 dense, G = 1, pages of 32
    (10, 2, dict(lens=[3, 300, 901, 47], page_size=64, num_q_heads=16, num_kv_heads=8,
                 head_dim=128, kv_dtype="fp8")),                   # fp8 dense, G = 2
    (1, 2, dict(lens=[1, 700, 33], page_size=64, num_q_heads=32, num_kv_heads=8,
                head_dim=128)),                                    # one wave does it all
    # shares of the least size (4 units; segments of 1 - 7 blocks plus a start cost of 2
    # units), so share boundaries fall at every place in and around the start costs
    (146, 2, dict(lens=[32] * 6 + [96] * 6 + [65, 200, 33, 130], page_size=32, num_q_heads=32,
                  num_kv_heads=8, head_dim=128)),
    # the same with two waves per SIMD (MXFP4: start cost 4, least share 5 units)
    (168, 2, dict(lens=[32] * 6 + [96] * 6 + [65, 200, 33, 130], page_size=32, num_q_heads=32,
                  num_kv_heads=8, head_dim=128, kv_dtype="mxfp4")),
]


@pytest.mark.parametrize("waves,cfg,over", AUTO_WAVES)
def test_auto_decode_few_waves(gpu_lib, auto_waves, waves, cfg, over):
    """The balanced decode schedule with few waves (the test-only wave override): long shares that
    cross many segment boundaries and segments cut over several waves match the
    oracle, and a second call gives the same bits."""
    from tests.device_batch import DeviceBatch
    auto_waves(waves)
    wl = workloads.make(cfg, num_splits=0, **over)
    print(f"[case] auto waves={waves} cfg={cfg} {over}", flush=True)
    db = DeviceBatch(wl)
    db.fill_history()
    db.step()
    torch.cuda.synchronize()
    dec, lse, _, _ = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    assert_close(dec, ref[0], wl.kv_dtype, f"waves={waves}")
    assert_lse_close(lse, ref[1], wl.kv_dtype, f"waves={waves}")
    first = [db.out_dec.clone(), db.lse_dec.clone()]
    db.decode_step()
    torch.cuda.synchronize()
    assert torch.equal(first[0].view(torch.int16), db.out_dec.view(torch.int16))
    assert torch.equal(first[1].view(torch.int32), db.lse_dec.view(torch.int32))


SHORT_CHUNKS = [
    # (waves (0 = device), page_size, chunks, cached, num_q_heads, num_kv_heads, head_dim):
    # chunks of at most 16 / G queries run on the balanced decode kernels
    (0, 64, [1, 2, 3, 4, 4, 2, 1], [100, 700, 2000, 64, 33, 4000, 5], 32, 8, 128),   # G = 4
    (0, 16, [2, 1, 2], [300, 17, 1000], 64, 8, 128),                              # G = 8, pages of 16
    (0, 32, [8, 5, 1, 7], [40, 300, 1200, 0], 16, 8, 64),                          # G = 2, D = 64
    (0, 128, [16, 3, 9], [129, 500, 31], 8, 8, 128),                               # G = 1, 16 queries
    (7, 64, [4, 4, 3, 1, 2], [3000, 800, 64, 1500, 90], 32, 8, 128),               # few waves: cut segments
    # 300 sequences: past the first 256, whose lengths and query rows each wave of the
    # balanced kernel keeps in registers, they are read from memory
    (0, 32, np.random.RandomState(300).randint(1, 5, 300).tolist(),
     np.random.RandomState(301).randint(0, 400, 300).tolist(), 32, 8, 128),
]


@pytest.mark.parametrize("waves,P,chunks,cached,hq,hkv,D", SHORT_CHUNKS)
def test_short_chunks_via_decode_kernels(gpu_lib, auto_waves, waves, P, chunks, cached, hq, hkv, D):
    """Prefill chunks of at most 16 / G queries (several tokens verified per sequence,
    as in speculative decoding) through paged_attn_prefill_chunk: all queries of a
    (sequence, kv head) share one MFMA tile of the decode kernels, each row with its
    causal limit; ragged chunk lengths, cut segments, every G that allows two or more
    queries per tile."""
    from paged_kv_cache_413_amd import binding as B
    from tests.device_batch import DeviceBatch
    if waves:
        auto_waves(waves)
    wl = workloads.make(3, num_seqs=0, num_prefill=len(chunks), prefill_chunk=chunks, prefill_cached=cached,
                        page_size=P, num_q_heads=hq, num_kv_heads=hkv, head_dim=D)
    print(f"[case] short chunks waves={waves} P={P} chunks={chunks} Hq={hq} Hkv={hkv} D={D}", flush=True)
    db = DeviceBatch(wl)
    db.fill_history()
    db.prepare_step()
    # the decode-kernel plan: its workspace is the balanced decode schedule's, with
    # 16-row records (differs from the query-tiled prefill plan's)
    ws = B.paged_attn_prefill_workspace_size(db.cache, db.seqs_pf, db.q_code, hq, db.npf_q, db.max_q)
    assert ws > 0
    db.step()
    torch.cuda.synchronize()
    _, _, pf, pf_lse = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    assert_close(pf, ref[2], "bf16", f"chunks={chunks}")
    assert_lse_close(pf_lse, ref[3], "bf16", f"chunks={chunks}")


PREFILL_EDGES = [
    # (page_size, chunks, cached, num_q_heads, num_kv_heads, head_dim)
    (64, [1, 15, 16, 17], [0, 0, 5, 100], 32, 8, 128),       # first chunks: triangular
    (64, [70, 64, 3], [190, 0, 4000], 32, 8, 128),
    (128, [33, 130], [0, 257], 16, 16, 64),                   # G = 1, D = 64
    (32, [40, 9], [31, 300], 16, 8, 128),                     # G = 2
    (16, [25, 50], [7, 100], 64, 8, 128),                     # G = 8, pages of 16
    (8, [20, 3], [13, 60], 32, 2, 64),                        # G = 16, pages of 8
    (64, [300, 5], [600, 2000], 32, 8, 128),                  # several query waves
    # chunks of at most two waves' queries (a wave holds 2 tiles x 16/G queries for
    # D = 128, 4 tiles for D = 64) run on the per-wave kernel with pages of >= 32 too
    (64, [5, 8, 7, 6], [100, 700, 2000, 64], 32, 8, 128),     # G = 4: 8 verified tokens
    (64, [16, 12, 9], [300, 1000, 40], 32, 8, 128),           # G = 4: two query tiles
    (128, [20, 32, 9], [0, 257, 1000], 16, 16, 128),          # G = 1: up to 32 queries
    (32, [12, 16], [33, 400], 16, 4, 64),                     # G = 4, D = 64: up to 16
]


@pytest.mark.parametrize("P,chunks,cached,hq,hkv,D", PREFILL_EDGES)
def test_prefill_edge_shapes(gpu_lib, P, chunks, cached, hq, hkv, D):
    """Causal prefill chunks on the matrix cores: first chunks (no cache, triangular
    masks), chunks of 1 and around the 16-row tile and 32-key block edges, groups of
    1..16 query heads, head_dim 64 and 128, pages of 8..128, and enough queries for
    several waves per (sequence, kv head) and for key splits to be merged."""
    from tests.device_batch import DeviceBatch
    wl = workloads.make(3, num_seqs=len(chunks) + 2, num_prefill=len(chunks), prefill_chunk=chunks,
                        prefill_cached=cached, median=50, clip=(1, 300), page_size=P,
                        num_q_heads=hq, num_kv_heads=hkv, head_dim=D)
    print(f"[case] prefill edge P={P} chunks={chunks} cached={cached} Hq={hq} Hkv={hkv} D={D}", flush=True)
    db = DeviceBatch(wl)
    db.fill_history()
    db.step()
    torch.cuda.synchronize()
    dec, dec_lse, pf, pf_lse = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    assert_close(pf, ref[2], "bf16", f"prefill P={P}")
    assert_lse_close(pf_lse, ref[3], "bf16", f"prefill P={P}")
    assert_close(dec, ref[0], "bf16", f"decode P={P}")


@pytest.mark.parametrize("chunks", [[70, 9], [2, 4, 1]])
def test_step_replays_from_a_captured_graph(gpu_lib, chunks):
    """A whole step (kv_append, prefill-chunk attention, decode attention and their
    merges) captured in a HIP graph and replayed three times, with eager kernels that
    overwrite every output in between: each replay reproduces the eager results bit for
    bit and matches the oracle (the library allocates nothing and enqueues no memset,
    so the step captures as is).  Query-tiled prefill chunks and short chunks on the decode kernels."""
    from tests.device_batch import DeviceBatch
    wl = workloads.make(3, num_seqs=6, num_prefill=len(chunks), prefill_chunk=chunks,
                        prefill_cached=[190, 40, 700][:len(chunks)], median=300, clip=(1, 900))
    print(f"[case] graph replay chunks={chunks}", flush=True)
    ref_pool = oracle_pool(wl)
    ref = oracle_outputs(wl, ref_pool)
    db = DeviceBatch(wl)
    db.fill_history()
    db.prepare_step()
    outs = [db.out_dec, db.lse_dec, db.out_pf, db.lse_pf]
    bits = lambda t: t.view(torch.int16) if t.dtype != torch.float32 else t.view(torch.int32)
    db.step()
    torch.cuda.synchronize()
    eager = [bits(t).clone() for t in outs]
    pool_eager = db.pool.view(torch.int16).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        db.step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        db.step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("decode out", "decode lse", "prefill out", "prefill lse"), outs, eager):
            assert torch.equal(bits(t), e), f"replay {rep}: {name}"
        assert torch.equal(db.pool.view(torch.int16), pool_eager), f"replay {rep}: pool"
        # and each replay's results against the oracle, not only against the eager run
        dec, dec_lse, pf, pf_lse = db.outputs_f64()
        assert_close(dec, ref[0], wl.kv_dtype, f"replay {rep}: decode")
        assert_lse_close(dec_lse, ref[1], wl.kv_dtype, f"replay {rep}: decode")
        assert_close(pf, ref[2], wl.kv_dtype, f"replay {rep}: prefill")
        assert_lse_close(pf_lse, ref[3], wl.kv_dtype, f"replay {rep}: prefill")
        assert np.array_equal(pool_token_major(db.pool_bits()).view(np.uint8), ref_pool.view(np.uint8)), \
            f"replay {rep}: pool differs from the oracle's"


WINDOWS = [
    # (workload, overrides, window W): every kernel family under a limited attention window
    (2, dict(num_seqs=7, len_range=(1, 700)), 1),                                  # decode, W = 1
    (2, dict(num_seqs=7, len_range=(1, 700)), 100),                                # balanced decode
    (2, dict(num_seqs=7, len_range=(1, 700), num_splits=3), 64),                   # fixed partitions
    (2, dict(lens=[5, 40, 333, 1000], page_size=16, num_q_heads=16, num_kv_heads=2, head_dim=64), 77),
    (5, dict(num_seqs=6, group_size=3, prefix_len=128, len_range=(129, 600)), 200),  # FP8, shared prefix
    (2, dict(num_seqs=140, len_range=(1, 300), kv_dtype="fp8"), 100),             # FP8, 1 120 segments: dense decode
    (1, dict(), 20),                                                               # f32: vector-ALU kernels
    (3, dict(num_seqs=9, num_prefill=2, prefill_chunk=70, prefill_cached=190, median=60, clip=(1, 400)), 50),
    (3, dict(num_seqs=0, num_prefill=5, prefill_chunk=[4, 1, 3, 4, 2],
             prefill_cached=[300, 40, 900, 64, 1000]), 33),                        # short chunks, decode kernels
    (3, dict(num_seqs=2, num_prefill=2, prefill_chunk=[40, 9], prefill_cached=[31, 300], page_size=16), 25),
    (3, dict(num_seqs=2, num_prefill=3, prefill_chunk=[16, 7, 12], prefill_cached=[500, 90, 1200]), 60),
    # ^ chunks of 5..16 queries on pages of 64: the per-wave prefill kernel
]


@pytest.mark.parametrize("cfg,over,W", WINDOWS)
def test_window_matches_oracle_after_page_release(gpu_lib, cfg, over, W):
    """A limited attention window W (a query at p sees keys p - W + 1 .. p) on every
    kernel family; before the attention calls, the pages no window reaches any more
    are released: their table entries set to -1 and their contents overwritten with
    NaN.  The result still matches the oracle: nothing before a window is read."""
    from paged_kv_cache_413_amd import page_table
    from tests.device_batch import DeviceBatch
    wl = workloads.make(cfg, window=W, **over)
    print(f"[case] window W={W} cfg={cfg} {over}", flush=True)
    db = DeviceBatch(wl)
    db.fill_history()
    db.prepare_step()
    db.append_step()
    torch.cuda.synchronize()
    tables, freed = page_table.release_out_of_window(wl.block_tables, wl.context_lens, wl.new_lens, W,
                                                     wl.page_size)
    db.block_tables.copy_(torch.from_numpy(tables).to(db.dev))
    if freed.size:
        idx = torch.from_numpy(freed).to(db.dev)
        if db.pool.dtype == torch.uint8:
            db.pool[idx] = 0x7F                     # the E4M3 NaN code
        else:
            db.pool[idx] = float("nan")
    db.prefill_step()
    db.decode_step()
    torch.cuda.synchronize()
    dec, dlse, pf, plse = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    if wl.num_prefill < wl.num_seqs:
        assert_close(dec, ref[0], wl.kv_dtype, f"W={W}")
        assert_lse_close(dlse, ref[1], wl.kv_dtype, f"W={W}")
    if wl.num_prefill:
        assert_close(pf, ref[2], wl.kv_dtype, f"W={W} prefill")
        assert_lse_close(plse, ref[3], wl.kv_dtype, f"W={W} prefill")


@pytest.mark.parametrize("P", [16, 64])
def test_prefix_reuse_with_partial_page_copy(gpu_lib, P):
    """Cross-request reuse: request B shares A's first 40 tokens.  The prefix index
    hands B A's full pages (shared through B's block table) and A's partly matching
    page, which kv_copy_pages copies into a page of B's own before B appends the rest
    of its tokens.  Decode of A and B then equals the oracle over unshared pages, and
    the copied page is A's page byte for byte."""
    from paged_kv_cache_413_amd import binding as B
    from paged_kv_cache_413_amd.prefix_index import PrefixIndex
    rng = np.random.default_rng(11)
    Hkv, Hq, D, share, La, Lb = 2, 8, 128, 40, 150, 120
    to_bf16 = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    ka, va = to_bf16(rng.standard_normal((La, Hkv, D))), to_bf16(rng.standard_normal((La, Hkv, D)))
    kb = torch.cat([ka[:share], to_bf16(rng.standard_normal((Lb - share, Hkv, D)))])
    vb = torch.cat([va[:share], to_bf16(rng.standard_normal((Lb - share, Hkv, D)))])
    tok_a = rng.integers(0, 1000, La).tolist()
    tok_b = tok_a[:share] + rng.integers(1000, 2000, Lb - share).tolist()
    npages = 64
    free = rng.permutation(npages).tolist()
    pages_a = [free.pop() for _ in range(-(-La // P))]
    dev = "cuda"
    pool = torch.full((npages, 2, Hkv, P, D), float("nan"), dtype=torch.bfloat16, device=dev)
    cache = B.make_cache(pool, P, Hkv, D, B.PKV_BF16)

    def run_append(table, L, k, v):
        bt = torch.tensor([table], dtype=torch.int32, device=dev)
        ctx = torch.tensor([L], dtype=torch.int32, device=dev)
        cu = torch.tensor([0, k.shape[0]], dtype=torch.int32, device=dev)
        B.kv_append(cache, B.make_seqs(bt, ctx, L), k.to(dev).contiguous(), v.to(dev).contiguous(), cu, k.shape[0])

    run_append(pages_a, La, ka, va)                      # A's history
    idx = PrefixIndex(P)
    idx.insert(tok_a, pages_a)
    m = idx.match(tok_b)
    assert m.pages == pages_a[:share // P] and m.partial_tokens == share % P
    assert m.partial_page == pages_a[share // P]
    pages_b = m.pages + [free.pop() for _ in range(-(-Lb // P) - len(m.pages))]
    src = torch.tensor([m.partial_page], dtype=torch.int32, device=dev)
    dst = torch.tensor([pages_b[len(m.pages)]], dtype=torch.int32, device=dev)
    B.kv_copy_pages(cache, src, dst, 1)
    torch.cuda.synchronize()
    assert torch.equal(pool[dst[0]].view(torch.int16), pool[src[0]].view(torch.int16))
    start = len(m.pages) * P + m.partial_tokens          # B's first token not yet cached
    run_append(pages_b, Lb, kb[start:], vb[start:])      # B's own tokens
    # decode of both (their last tokens are this step's)
    q = to_bf16(rng.standard_normal((2, Hq, D)))
    width = max(len(pages_a), len(pages_b))
    bt = torch.full((2, width), -1, dtype=torch.int32)
    bt[0, :len(pages_a)] = torch.tensor(pages_a)
    bt[1, :len(pages_b)] = torch.tensor(pages_b)
    bt, ctx = bt.to(dev), torch.tensor([La, Lb], dtype=torch.int32, device=dev)
    seqs = B.make_seqs(bt, ctx, La)
    out = torch.empty((2, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((2, Hq), dtype=torch.float32, device=dev)
    ws_n = B.paged_attn_decode_workspace_size(cache, seqs, B.PKV_BF16, Hq, 0)
    ws = torch.zeros(max(ws_n, 1), dtype=torch.uint8, device=dev)
    B.paged_attn_decode(cache, seqs, q.to(dev), B.PKV_BF16, Hq, 1.0 / np.sqrt(D), 0, out, lse, ws, ws_n)
    torch.cuda.synchronize()
    # oracle: the same logical tokens in unshared pages
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    opool = oracle.new_pool(2 * width, Hkv, P, D, "bf16", fill=0x7FC0)
    otab = np.full((2, width), -1, np.int32)
    otab[0, :len(pages_a)] = np.arange(len(pages_a))
    otab[1, :len(pages_b)] = width + np.arange(len(pages_b))
    oracle.append(opool, otab, np.array([La, Lb]), np.array([La, Lb]),
                  np.concatenate([bits(ka), bits(kb)]), np.concatenate([bits(va), bits(vb)]), "bf16", "bf16")
    ref_o, ref_l = oracle.decode(opool, otab, np.array([La, Lb]), bits(q), "bf16", np.float32(1.0 / np.sqrt(D)), "bf16")
    assert_close(out.float().cpu().numpy().astype(np.float64), ref_o, "bf16", f"P={P}")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_l, "bf16", f"P={P}")


FP8_PREFILL = [
    # (page_size, chunks, cached, num_q_heads, num_kv_heads, head_dim, window)
    (64, [70, 200], [190, 1000], 32, 8, 128, 0),       # LDS-shared prefill kernel
    (16, [40, 9], [31, 300], 64, 8, 128, 0),           # per-wave kernel (pages of 16), G = 8
    (64, [4, 3, 1], [500, 64, 2000], 32, 8, 128, 0),   # short chunks: decode kernels
    (128, [100, 33], [0, 700], 16, 8, 64, 90),         # D = 64, G = 2, window
    (64, [8, 6, 5], [300, 1000, 40], 32, 8, 128, 0),   # per-wave kernel, pages of 64
]


@pytest.mark.parametrize("P,chunks,cached,hq,hkv,D,W", FP8_PREFILL)
def test_fp8_prefill_matches_oracle(gpu_lib, P, chunks, cached, hq, hkv, D, W):
    """Prefill-chunk attention over an FP8 (E4M3) cache with per-kv-head scales, on
    each prefill path, decode rows in the same batch."""
    from tests.device_batch import DeviceBatch
    wl = workloads.make(3, num_seqs=4, num_prefill=len(chunks), prefill_chunk=chunks, prefill_cached=cached,
                        median=200, clip=(1, 600), page_size=P, num_q_heads=hq, num_kv_heads=hkv,
                        head_dim=D, kv_dtype="fp8", window=W)
    print(f"[case] fp8 prefill P={P} chunks={chunks} Hq={hq} Hkv={hkv} D={D} W={W}", flush=True)
    db = DeviceBatch(wl)
    db.fill_history()
    db.step()
    torch.cuda.synchronize()
    dec, dlse, pf, plse = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    assert_close(pf, ref[2], "fp8", f"chunks={chunks}")
    assert_lse_close(plse, ref[3], "fp8", f"chunks={chunks}")
    assert_close(dec, ref[0], "fp8", "decode rows")
    assert_lse_close(dlse, ref[1], "fp8", "decode rows")
