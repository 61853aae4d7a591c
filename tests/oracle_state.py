"""Builds the oracle's page pool for a workload (test infrastructure).

The pool starts as NaN everywhere, pages named by a block table are then filled with
the poison value, and the workload's history and (optionally) this step's tokens are
appended with the oracle's own append."""
import numpy as np

import oracle
import workloads


def scales(wl):
    if wl.kv_dtype != "fp8":
        return None, None, None, None
    return wl.fp8_scales()


def oracle_pool(wl, include_step=True):
    nan, poison = workloads.fill_bits(wl.kv_dtype)
    pool = oracle.new_pool(wl.num_pages, wl.num_kv_heads, wl.page_size, wl.head_dim,
                           wl.kv_dtype, fill=nan)
    pool[wl.referenced_pages()] = poison
    ks, vs, kinv, vinv = scales(wl)
    for rows, ctx, new, k, v in wl.history_plan():
        oracle.append(pool, wl.block_tables[rows], ctx, new, k, v, wl.in_dtype, wl.kv_dtype,
                      kinv, vinv)
    if include_step:
        k, v = wl.step_kv()
        oracle.append(pool, wl.block_tables, wl.context_lens, wl.new_lens, k, v, wl.in_dtype,
                      wl.kv_dtype, kinv, vinv)
    return pool


def oracle_outputs(wl, pool):
    """(decode_out, decode_lse, prefill_out, prefill_lse) for the workload, float64.
    Decode covers sequences [num_prefill, S); prefill covers [0, num_prefill)."""
    ks, vs, _, _ = scales(wl)
    q = wl.q_packed()
    npf = wl.num_prefill
    cu = wl.cu(wl.new_lens)
    pf = (None, None)
    if npf:
        pf = oracle.prefill_chunk(pool, wl.block_tables[:npf], wl.context_lens[:npf],
                                  cu[:npf + 1], q[:cu[npf]], wl.q_dtype, wl.sm_scale,
                                  wl.kv_dtype, ks, vs, window=wl.window)
    dq = q[cu[npf]:]
    dec = oracle.decode(pool, wl.block_tables[npf:], wl.context_lens[npf:], dq, wl.q_dtype,
                        wl.sm_scale, wl.kv_dtype, ks, vs, window=wl.window)
    return dec[0], dec[1], pf[0], pf[1]


def oracle_sequence(wl, s):
    """Oracle outputs of sequence s alone, from a compact pool holding only its pages
    (renumbered 0..n-1; the oracle's result does not depend on physical page ids).
    Returns (out [C][Hq][D], lse [C][Hq]) float64 for its C = new_lens[s] query rows:
    decode rows for a decode sequence, the causal chunk for a prefill request."""
    ks, vs, kinv, vinv = scales(wl)
    _, poison = workloads.fill_bits(wl.kv_dtype)
    row = wl.block_tables[s]
    n_used = int((row >= 0).sum())
    table = np.full((1, len(row)), -1, np.int32)
    table[0, :n_used] = np.arange(n_used, dtype=np.int32)
    pool = oracle.new_pool(n_used, wl.num_kv_heads, wl.page_size, wl.head_dim, wl.kv_dtype,
                           fill=poison)
    L, C = int(wl.context_lens[s]), int(wl.new_lens[s])
    k, v = wl.tokens(s, 0, L)
    oracle.append(pool, table, np.array([L]), np.array([L]), k, v, wl.in_dtype, wl.kv_dtype,
                  kinv, vinv)
    cu = wl.cu(wl.new_lens)
    q = wl.q_packed()[cu[s]:cu[s + 1]]
    if s < wl.num_prefill:
        return oracle.prefill_chunk(pool, table, np.array([L]), np.array([0, C]), q, wl.q_dtype,
                                    wl.sm_scale, wl.kv_dtype, ks, vs, window=wl.window)
    return oracle.decode(pool, table, np.array([L]), q, wl.q_dtype, wl.sm_scale, wl.kv_dtype,
                         ks, vs, window=wl.window)
