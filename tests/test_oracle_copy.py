"""Pin of the oracle's copy_pages (copy-on-partial-reuse) against facts fixed outside it.

Request B shares the first 40 tokens of request A ("NVIDIA TensorRT-LLM详解：架构、KV
Cache、调度与部署实践", §10 cross-request reuse and §11 partial reuse): B's block table
names A's two full pages, then a page of B's own into which copy_pages copies A's
partly matching page, then fresh pages; B appends its remaining tokens.  The pin:
decode attention of A and of B through the oracle's pool equals dense attention
(torch SDPA, float64) over the requests' *logical* K/V, which never pass through a
pool; the copied page is its source byte for byte and no other page changes.  A
planted mistake in the copy (V left behind, the wrong source page, no copy at all)
must fail the pin.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

HKV, HQ, D, P = 2, 4, 64, 16
LA, LB, SHARE = 70, 57, 40           # B matches 2 full pages + 8 tokens of A's page 2


def _bf16_bits(x):
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _case(kv_dtype, seed=5):
    rng = np.random.default_rng(seed)
    ka = _bf16_bits(rng.standard_normal((LA, HKV, D)))
    va = _bf16_bits(rng.standard_normal((LA, HKV, D)))
    kb = np.concatenate([ka[:SHARE], _bf16_bits(rng.standard_normal((LB - SHARE, HKV, D)))])
    vb = np.concatenate([va[:SHARE], _bf16_bits(rng.standard_normal((LB - SHARE, HKV, D)))])
    q = _bf16_bits(rng.standard_normal((2, HQ, D)))
    sc = (None,) * 4
    if kv_dtype == "fp8":
        amax = lambda x: torch.from_numpy(np.concatenate([x])).view(torch.bfloat16).double().abs().amax(dim=(0, 2)).numpy()
        ks = (np.maximum(amax(ka), amax(kb)) / 448.0).astype(np.float32)
        vs = (np.maximum(amax(va), amax(vb)) / 448.0).astype(np.float32)
        sc = (ks, vs, (1.0 / ks.astype(np.float64)).astype(np.float32),
              (1.0 / vs.astype(np.float64)).astype(np.float32))
    return ka, va, kb, vb, q, sc


def _logical(x, kv_dtype, scale):
    """bf16 rows [L][H][D] -> float64 through torch's casts (FP8: torch's E4M3 cast)."""
    t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()
    if kv_dtype == "fp8":
        inv = torch.from_numpy((1.0 / scale.astype(np.float64)).astype(np.float32))
        t = (t.float() * inv[None, :, None]).to(torch.float8_e4m3fn).double() * \
            torch.from_numpy(scale).double()[None, :, None]
    return t


def _sdpa(q, k, v, kv_dtype, ks, vs):
    G = HQ // HKV
    kk = _logical(k, kv_dtype, ks).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    vv = _logical(v, kv_dtype, vs).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    qq = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).double()[None, :, None, :]  # [1][Hq][1][D]
    o = F.scaled_dot_product_attention(qq, kk, vv, scale=float(np.float32(1 / np.sqrt(D))))
    return o[0, :, 0].numpy()


def _run(kv_dtype, copy_fn):
    ka, va, kb, vb, q, (ks, vs, kinv, vinv) = _case(kv_dtype)
    rng = np.random.default_rng(17)
    npages = 24
    free = rng.permutation(npages).tolist()
    nan = np.uint8(0x7F) if kv_dtype == "fp8" else np.uint16(0x7FC0)
    pool = oracle.new_pool(npages, HKV, P, D, kv_dtype, fill=nan)
    pages_a = [free.pop() for _ in range(-(-LA // P))]
    tab_a = np.array([pages_a], np.int32)
    oracle.append(pool, tab_a, np.array([LA]), np.array([LA]), ka, va, "bf16", kv_dtype, kinv, vinv)
    full = SHARE // P
    own = free.pop()
    pages_b = pages_a[:full] + [own] + [free.pop() for _ in range(-(-LB // P) - full - 1)]
    before = pool.copy()
    copy_fn(pool, [pages_a[full]], [own])
    copied = pool.copy()
    tab_b = np.array([pages_b], np.int32)
    start = SHARE                                    # B's first token not yet cached
    oracle.append(pool, tab_b, np.array([LB]), np.array([LB - start]), kb[start:], vb[start:],
                  "bf16", kv_dtype, kinv, vinv)
    width = max(len(pages_a), len(pages_b))
    tables = np.full((2, width), -1, np.int32)
    tables[0, :len(pages_a)], tables[1, :len(pages_b)] = pages_a, pages_b
    out, _ = oracle.decode(pool, tables, np.array([LA, LB]), q, "bf16",
                           np.float32(1 / np.sqrt(D)), kv_dtype, ks, vs)
    ref = np.stack([_sdpa(q[0], ka, va, kv_dtype, ks, vs), _sdpa(q[1], kb, vb, kv_dtype, ks, vs)])
    return out, ref, before, copied, pages_a[full], own


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_copy_on_partial_reuse_equals_dense_attention(kv_dtype):
    out, ref, before, copied, src, dst = _run(kv_dtype, oracle.copy_pages)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # the copy: the destination is its source byte for byte; nothing else moved
    assert np.array_equal(copied[dst].view(np.uint8), before[src].view(np.uint8))
    others = np.ones(len(before), bool)
    others[dst] = False
    assert np.array_equal(copied[others].view(np.uint8), before[others].view(np.uint8))


def _copy_k_only(pool, src, dst):
    for s, d in zip(src, dst):
        pool[int(d), 0] = pool[int(s), 0]


def _copy_next_page(pool, src, dst):
    for s, d in zip(src, dst):
        pool[int(d)] = pool[(int(s) + 1) % len(pool)]


def _no_copy(pool, src, dst):
    pass


@pytest.mark.parametrize("planted", [_copy_k_only, _copy_next_page, _no_copy])
def test_planted_copy_mistakes_fail_the_pin(planted):
    out, ref, *_ = _run("bf16", planted)
    bad = not np.isfinite(out).all() or not np.allclose(out, ref, rtol=0, atol=1e-6)
    assert bad, f"{planted.__name__} went unnoticed"
