"""Pins of the oracle's limited attention window against facts fixed outside it.

The reading ([Deep dive] §11, limited attention window: tokens outside a sliding window
take no further part in attention): a query at position p attends to keys p - W + 1 ..
p.  Checked by
* W1  dense attention (torch SDPA, float64) over logical tokens with a band mask built
      here, independently of the oracle's page gather and index shifts;
* W2  W = 1 is the closed form: the output is the V row at the query's own position,
      exactly, and the log-sum-exp is that one key's scaled logit;
* W3  W >= every context length gives the unwindowed result bit for bit;
* W4  pages that hold only keys before every window may hold anything (NaN here):
      nothing of them is read.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from tests.oracle_state import oracle_outputs, oracle_pool
from tests.test_oracle_attention import logical_f64, logical_kv

SMALL = {
    2: dict(num_seqs=5, len_range=(1, 300)),
    3: dict(num_seqs=6, num_prefill=2, prefill_chunk=70, prefill_cached=130, median=40, clip=(1, 200)),
    5: dict(num_seqs=6, group_size=3, prefix_len=128, len_range=(129, 400)),
}


def banded_sdpa(wl, W):
    q = logical_f64(wl, wl.q_packed())
    cu = wl.cu(wl.new_lens)
    G = wl.group_size
    out = torch.zeros_like(q)
    for s in range(wl.num_seqs):
        L, C = int(wl.context_lens[s]), int(wl.new_lens[s])
        k, v = logical_kv(wl, s)
        kr = k.repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
        vr = v.repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
        qs = q[cu[s]:cu[s + 1]].permute(1, 0, 2)[None]
        pos = torch.arange(L - C, L)[:, None]
        t = torch.arange(L)[None, :]
        mask = (t <= pos) & (t > pos - W)
        o = F.scaled_dot_product_attention(qs, kr, vr, attn_mask=mask, scale=float(np.float32(wl.sm_scale)))
        out[cu[s]:cu[s + 1]] = o[0].permute(1, 0, 2)
    return out.numpy()


def _outputs(wl):
    dec, dlse, pf, plse = oracle_outputs(wl, oracle_pool(wl))
    if wl.num_prefill:
        return np.concatenate([pf, dec]), np.concatenate([plse, dlse])
    return dec, dlse


@pytest.mark.parametrize("W", [1, 7, 32, 100])
@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_w1_window_equals_banded_dense_attention(cfg, W):
    wl = workloads.make(cfg, window=W, **SMALL[cfg])
    got, _ = _outputs(wl)
    np.testing.assert_allclose(got, banded_sdpa(wl, W), rtol=0, atol=1e-12)


@pytest.mark.parametrize("cfg", [2, 3])
def test_w2_window_of_one_returns_the_own_value_row(cfg):
    wl = workloads.make(cfg, window=1, **SMALL[cfg])
    got, lse = _outputs(wl)
    q = logical_f64(wl, wl.q_packed()).numpy()
    cu = wl.cu(wl.new_lens)
    G = wl.group_size
    for s in range(wl.num_seqs):
        L, C = int(wl.context_lens[s]), int(wl.new_lens[s])
        k, v = (x.numpy() for x in logical_kv(wl, s))
        for i in range(C):
            p, r = L - C + i, cu[s] + i
            want = np.repeat(v[p], G, axis=0)                     # [Hq][D]
            assert np.array_equal(got[r], want), (s, i)
            logit = np.float64(np.float32(wl.sm_scale)) * np.einsum("hd,hd->h", q[r], np.repeat(k[p], G, axis=0))
            np.testing.assert_allclose(lse[r], logit, rtol=0, atol=1e-9)


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_w3_window_covering_everything_is_full_attention(cfg):
    full = workloads.make(cfg, **SMALL[cfg])
    wide = workloads.make(cfg, window=int(full.context_lens.max()), **SMALL[cfg])
    a, b = _outputs(full), _outputs(wide)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_w4_pages_before_every_window_are_never_read():
    W = 40
    wl = workloads.make(2, window=W, num_seqs=4, len_range=(200, 300))
    pool = oracle_pool(wl)
    ref = oracle_outputs(wl, pool)
    P = wl.page_size
    poisoned = pool.copy()
    for s in range(wl.num_seqs):
        lo = int(wl.context_lens[s]) - W
        for i in range(lo // P):                                   # pages wholly before the window
            poisoned[wl.block_tables[s][i]] = np.nan if poisoned.dtype == np.float32 else 0x7FC0
    got = oracle_outputs(wl, poisoned)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def test_w1_catches_an_off_by_one_window(monkeypatch):
    """A plausible mistake (the window starting one key early) must fail the
    banded dense-attention pin."""
    wl = workloads.make(2, window=7, **SMALL[2])
    ref = banded_sdpa(wl, 7)
    real = oracle.paged_attention.window_start
    monkeypatch.setattr(oracle.paged_attention, "window_start", lambda pos, w: real(pos, w + 1))
    got, _ = _outputs(wl)
    assert np.abs(got - ref).max() > 1e-3
