"""GPU parity of the MXFP4 cache (OCP MX: E2M1 codes, an E8M0 scale per 32 dims of a
token row), through the C ABI: kv_append's encoding and the page gather bit for bit
against the oracle's MXFP4 codec, and decode / prefill attention element by element
against the oracle's fp64 attention over the decoded values."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_common import assert_close, assert_lse_close, mx_pool_logical, mx_unpack
from tests.oracle_state import oracle_outputs, oracle_pool

pytestmark = pytest.mark.gpu

CASES = {
    # Llama-shaped decode: D=128, G=4, pages of 64, ragged lengths 1..700
    "dec128": (2, dict(num_seqs=7, len_range=(1, 700), kv_dtype="mxfp4")),
    # D=64, G=8, pages of 32
    "dec64": (2, dict(num_seqs=5, len_range=(1, 400), kv_dtype="mxfp4", head_dim=64, num_q_heads=16,
                      num_kv_heads=2, page_size=32)),
    # two 70-token prefill chunks (the LDS-shared prefill kernel) and 7 decode sequences
    "mixed": (3, dict(num_seqs=7, num_prefill=2, prefill_chunk=70, prefill_cached=190, median=60,
                      clip=(1, 400), kv_dtype="mxfp4")),
    # chunks of 1, 3 and 4 tokens (at most 16 / G: the balanced decode kernels), odd and
    # even start positions, so both nibbles of shared V bytes are appended
    "short": (3, dict(num_seqs=4, num_prefill=3, prefill_chunk=[1, 3, 4], prefill_cached=[33, 64, 101],
                      median=50, clip=(1, 200), kv_dtype="mxfp4")),
    # the LDS-shared prefill kernel's MXFP4 staging at D = 64 (half the threads stage),
    # G = 8, pages of 32; and at D = 128, G = 16, pages of 128 with a first chunk
    "pf64": (3, dict(num_seqs=5, num_prefill=2, prefill_chunk=[40, 75], prefill_cached=[33, 100], median=50,
                     clip=(1, 200), kv_dtype="mxfp4", head_dim=64, num_q_heads=16, num_kv_heads=2, page_size=32)),
    # chunks of 5..8 queries at G = 4: the per-wave prefill kernel on pages of 64
    "mid": (3, dict(num_seqs=3, num_prefill=3, prefill_chunk=[8, 6, 5], prefill_cached=[300, 64, 1000],
                    median=60, clip=(1, 300), kv_dtype="mxfp4")),
    "pf_g16": (3, dict(num_seqs=4, num_prefill=2, prefill_chunk=[64, 23], prefill_cached=[0, 250], median=60,
                       clip=(1, 300), kv_dtype="mxfp4", num_q_heads=32, num_kv_heads=2, page_size=128)),
}


def _batch(name, num_splits=None, **extra):
    from tests.device_batch import DeviceBatch
    cfg, over = CASES[name]
    wl = workloads.make(cfg, **{**over, **extra})
    print(f"[case] mxfp4 {name} S={wl.num_seqs} Lmax={wl.max_context_len} D={wl.head_dim} "
          f"P={wl.page_size} window={wl.window}", flush=True)
    db = DeviceBatch(wl, num_splits=num_splits)
    db.fill_history()
    db.prepare_step()
    return wl, db


def _written(wl):
    """Mask [pages][P] of the slots that hold a token after this step's append."""
    m = np.zeros((wl.num_pages, wl.page_size), bool)
    for s in range(wl.num_seqs):
        t = np.arange(int(wl.context_lens[s]))
        m[wl.block_tables[s][t // wl.page_size], t % wl.page_size] = True
    return m


@pytest.mark.parametrize("name", list(CASES))
def test_mx_append_is_bit_exact(gpu_lib, name):
    """Every cached token row equals the oracle's encoding, codes and scales; every
    other slot still holds the bytes the pool was filled with."""
    wl, db = _batch(name)
    db.append_step()
    torch.cuda.synchronize()
    P, D = wl.page_size, wl.head_dim
    got = mx_pool_logical(db.pool_bits(), P, D)
    ref = oracle_pool(wl)
    assert got.shape == ref.shape
    w = _written(wl)
    gw, rw = got.transpose(0, 3, 1, 2, 4)[w], ref.transpose(0, 3, 1, 2, 4)[w]
    assert np.array_equal(gw, rw), f"{int((gw != rw).sum())} of {gw.size} entries differ"
    nan, poison = workloads.fill_bits("mxfp4")
    fill = np.full(db.pool.shape, nan, np.uint8)
    fill[wl.referenced_pages()] = poison
    fl = mx_pool_logical(fill, P, D).transpose(0, 3, 1, 2, 4)
    assert np.array_equal(got.transpose(0, 3, 1, 2, 4)[~w], fl[~w])


@pytest.mark.parametrize("name", ["dec128", "dec64"])
def test_mx_debug_gather_is_bit_exact(gpu_lib, name):
    from paged_kv_cache_413_amd import binding as B
    wl, db = _batch(name)
    db.append_step()
    S, Lm, H, D = wl.num_seqs, wl.max_context_len, wl.num_kv_heads, wl.head_dim
    row = D // 2 + D // 32
    kout = torch.zeros((S, Lm, H, row), dtype=torch.uint8, device=db.dev)
    vout = torch.zeros_like(kout)
    B.paged_kv_debug_gather(db.cache, db.seqs_all, kout, vout)
    torch.cuda.synchronize()
    kg, vg = kout.cpu().numpy(), vout.cpu().numpy()
    for s in range(S):
        L = int(wl.context_lens[s])
        k, v = wl.tokens(s)
        for x, got in ((k, kg[s, :L]), (v, vg[s, :L])):
            codes, scales = oracle.mx_encode(oracle.paged_attention.to_f64(x, "bf16"))
            assert np.array_equal(mx_unpack(got[..., :D // 2]), codes)
            assert np.array_equal(got[..., D // 2:], scales)
        assert (kg[s, L:] == 0).all() and (vg[s, L:] == 0).all()


@pytest.mark.parametrize("name", list(CASES))
def test_mx_attention_matches_oracle(gpu_lib, name):
    wl, db = _batch(name)
    db.step()
    torch.cuda.synchronize()
    dec, dec_lse, pf, pf_lse = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    err = assert_close(dec, ref[0], "mxfp4", "decode")
    assert_lse_close(dec_lse, ref[1], "mxfp4", "decode")
    if wl.num_prefill:
        assert_close(pf, ref[2], "mxfp4", "prefill")
        assert_lse_close(pf_lse, ref[3], "mxfp4", "prefill")
    print(f"[ok] mxfp4 {name} decode err {err:.3e}", flush=True)


@pytest.mark.parametrize("splits", [2, 5])
def test_mx_fixed_partitions(gpu_lib, splits):
    wl, db = _batch("dec128", num_splits=splits)
    db.step()
    torch.cuda.synchronize()
    dec, lse, _, _ = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    assert_close(dec, ref[0], "mxfp4", f"splits={splits}")
    assert_lse_close(lse, ref[1], "mxfp4", f"splits={splits}")


@pytest.mark.parametrize("waves", [3, 37])
def test_mx_few_waves(gpu_lib, auto_waves, waves):
    """Balanced schedule with few waves: shares cut (sequence, kv head) segments
    mid-page, merged by the merge kernel."""
    auto_waves(waves)
    wl, db = _batch("mixed")
    db.step()
    torch.cuda.synchronize()
    dec, lse, pf, pf_lse = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    assert_close(dec, ref[0], "mxfp4", f"waves={waves}")
    assert_lse_close(lse, ref[1], "mxfp4", f"waves={waves}")
    assert_close(pf, ref[2], "mxfp4", f"waves={waves} prefill")


@pytest.mark.parametrize("name,window", [("mixed", 50), ("short", 40), ("dec64", 97)])
def test_mx_window(gpu_lib, name, window):
    wl, db = _batch(name, window=window)
    db.step()
    torch.cuda.synchronize()
    dec, lse, pf, pf_lse = db.outputs_f64()
    ref = oracle_outputs(wl, oracle_pool(wl))
    assert_close(dec, ref[0], "mxfp4", f"window={window}")
    assert_lse_close(lse, ref[1], "mxfp4", f"window={window}")
    if wl.num_prefill:
        assert_close(pf, ref[2], "mxfp4", f"window={window} prefill")


def _edge_blocks(rng, n):
    """n blocks of 32 bf16 values (as float32, exactly representable) that reach the
    encoder's edges: exact midpoints of the E2M1 grid (ties to even), magnitudes above
    6 X (clamped), zeros and negative zeros, blocks of bf16 subnormals (scale byte 0),
    subnormals beside a small normal maximum, values near the bf16 maximum (scale
    byte 252), and plain N(0, 1) values."""
    out = np.empty((n, 32), np.float32)
    ties = np.array([6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, .5, 1, 1.5, 2, 3, 4, 0, 0.125])
    for i in range(n):
        kind, k = i % 7, int(rng.integers(-20, 20))
        if kind == 0:
            v = rng.permutation(np.concatenate([ties, -ties])) * 2.0 ** k
        elif kind == 1:
            v = rng.choice([7.5, 7.0, 6.5, 6.25, 5.5, 0.3, -7.75, 1.0], 32) * 2.0 ** k
        elif kind == 2:
            v = np.where(rng.random(32) < .5, -0.0, 0.0)
        elif kind == 3:
            v = rng.integers(-127, 128, 32) * 2.0 ** -133
        elif kind == 4:
            v = rng.integers(-127, 128, 32) * 2.0 ** -133
            v[int(rng.integers(32))] = 2.0 ** -124
        elif kind == 5:
            v = rng.choice([3.3e38, -3.0e38, 1.7e38, 2.5e37, 1.0], 32)
        else:
            v = rng.standard_normal(32)
        b = (np.asarray(v, np.float32).view(np.uint32) + 0x8000) >> 16   # to bf16 (near), then back
        out[i] = (b.astype(np.uint32) << 16).view(np.float32)
    return out


def test_mx_append_encodes_edge_values(gpu_lib):
    """kv_append into an MXFP4 cache, bit for bit against the oracle's codec, on blocks
    built to hit every rounding, clamping and scale edge of the encoding."""
    from paged_kv_cache_413_amd import binding as B
    rng = np.random.default_rng(4130)
    T, H, D, P = 32, 2, 64, 32
    print(f"[case] mxfp4 append edges T={T} H={H} D={D}", flush=True)
    tile = B.paged_kv_page_bytes(B.PKV_MXFP4, P, H, D) // (2 * H)
    pool = torch.zeros((1, 2, H, tile), dtype=torch.uint8, device="cuda")
    cache = B.make_cache(pool, P, H, D, B.PKV_MXFP4)
    table = torch.zeros((1, 1), dtype=torch.int32, device="cuda")       # page 0
    lens = torch.full((1,), T, dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    seqs = B.make_seqs(table, lens, T)
    vals = {kv: _edge_blocks(rng, T * H * D // 32).reshape(T, H, D) for kv in ("k", "v")}
    dev = {kv: torch.from_numpy(x).to("cuda").to(torch.bfloat16) for kv, x in vals.items()}
    torch.cuda.synchronize()
    assert int(table.max()) == 0 and int(lens[0]) == T, "table or lengths changed"
    B.kv_append(cache, seqs, dev["k"], dev["v"], cu, T)
    row = D // 2 + D // 32
    kout = torch.zeros((1, T, H, row), dtype=torch.uint8, device="cuda")
    vout = torch.zeros_like(kout)
    B.paged_kv_debug_gather(cache, seqs, kout, vout)
    torch.cuda.synchronize()
    for kv, got in (("k", kout), ("v", vout)):
        codes, scales = oracle.mx_encode(vals[kv].astype(np.float64))
        g = got[0].cpu().numpy()
        assert np.array_equal(mx_unpack(g[..., :D // 2]), codes), f"{kv} codes differ"
        assert np.array_equal(g[..., D // 2:], scales), f"{kv} scales differ"
