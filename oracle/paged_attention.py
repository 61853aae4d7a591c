"""Paged-KV attention, written as its plain definition in float64.  Test infrastructure.

Pages cited (by title):
  [Deep dive]  "NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践"
  [Concept]    "TensorRT-LLM" (concept explainer)

Cache layout (one layer): pool[page][kv][kv_head][slot][dim], kv = 0 for K and 1 for
V.  A page holds `page_size` consecutive tokens of one sequence; the block table of a
sequence maps its logical page i to a physical page ([Deep dive] §9, the figure that
maps logical blocks 0,1,2 to physical blocks 17,3,91; [Concept] 关键机制,
PagedAttention: fixed-size pages, a page table from logical position to physical
memory, pages allocated as the sequence grows).  The pages leave the order inside a
page open; this is the paged form of the contiguous cache
[batch*beam][2][heads][max_seq_len][head_dim] that [Deep dive] §9 shows, with the
sequence axis cut into pages.

Storage dtypes: "f32" (float32), "bf16" (bit patterns in uint16), "fp8" (OCP E4M3
codes in uint8, with one float32 dequantization scale per kv head for K and for V),
"mxfp4" (OCP MXFP4: a row is stored as its D E2M1 codes, one per byte, then its D/32
E8M0 block scales, so the last pool axis has D + D/32 entries).

Query head h reads kv head h // G, G = Hq / Hkv (consecutive query heads share a KV
head; the pages do not fix the grouping and this is the plainest reading).
"""
from __future__ import annotations

import numpy as np

from .fp8_e4m3 import decode_e4m3, encode_e4m3
from .mxfp4 import mx_decode, mx_encode

STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "mxfp4": np.uint8}


def new_pool(num_pages, num_kv_heads, page_size, head_dim, kv_dtype, fill=0):
    """A pool of `num_pages` pages filled with the storage value `fill`."""
    row = head_dim + head_dim // 32 if kv_dtype == "mxfp4" else head_dim
    return np.full((num_pages, 2, num_kv_heads, page_size, row), fill,
                   dtype=STORAGE[kv_dtype])


def slot_of(block_table_row, t: int, page_size: int):
    """(physical page, slot) that holds logical token t ([Deep dive] §9 figure)."""
    return int(block_table_row[t // page_size]), t % page_size


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Storage values -> float64 (exact for f32 and bf16)."""
    if dtype == "f32":
        return np.asarray(bits, np.float32).astype(np.float64)
    if dtype == "bf16":
        u32 = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):       # NaN patterns stay NaN
            return u32.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def encode_rows(x: np.ndarray, in_dtype: str, kv_dtype: str, inv_scale=None) -> np.ndarray:
    """Encode K or V rows [..., Hkv, D] of the input dtype into the cache dtype.

    f32 and bf16 caches store the input bits unchanged.  An FP8 cache stores
    e4m3(f32(x * inv_scale[h])): the product of a bf16 and a float32 is exact in
    float64, so rounding it to float32 is one IEEE float32 multiply, followed by one
    round-to-nearest-even into E4M3 with saturation ([Deep dive] §13, FP8 KV cache)."""
    if kv_dtype == in_dtype:
        return np.array(x, dtype=STORAGE[kv_dtype], copy=True)
    if kv_dtype == "fp8" and in_dtype == "bf16":
        inv = np.asarray(inv_scale, np.float32).astype(np.float64)
        prod = to_f64(x, "bf16") * inv[:, None]
        return encode_e4m3(prod.astype(np.float32))
    if kv_dtype == "mxfp4" and in_dtype == "bf16":
        # each row's 32-element blocks along D are encoded by themselves
        codes, scales = mx_encode(to_f64(x, "bf16"))
        return np.concatenate([codes, scales], axis=-1)
    raise ValueError(f"cannot store {in_dtype} in a {kv_dtype} cache")


def append(pool, block_tables, context_lens, new_lens, k_new, v_new, in_dtype, kv_dtype,
           k_inv_scale=None, v_inv_scale=None):
    """Write each new token's K/V into the slot its block table names.

    Sequence s appends new_lens[s] tokens at positions context_lens[s] - new_lens[s]
    ... context_lens[s] - 1 (context_lens counts the tokens in the cache after the
    append); its rows sit consecutively in the packed k_new / v_new [total][Hkv][D],
    sequences in order.  A decode step writes one new token per sequence
    ([Deep dive] §2, decode outline); a prefill chunk writes the whole chunk
    ([Deep dive] §8).  Returns the written (page, slot) pairs in order."""
    P = pool.shape[3]
    written = []
    row = 0
    for s in range(len(context_lens)):
        L, n = int(context_lens[s]), int(new_lens[s])
        pos = np.arange(L - n, L)
        pages = block_tables[s][pos // P]
        slots = pos % P
        pool[pages, 0, :, slots, :] = encode_rows(k_new[row:row + n], in_dtype, kv_dtype, k_inv_scale)
        pool[pages, 1, :, slots, :] = encode_rows(v_new[row:row + n], in_dtype, kv_dtype, v_inv_scale)
        written.extend(zip(pages.tolist(), slots.tolist()))
        row += n
    return written


def copy_pages(pool, src_pages, dst_pages):
    """Page dst[i] becomes a copy of page src[i] (all of its K and V), for every i:
    copy-on-partial-reuse gives a request that matches only the first tokens of a
    cached block a block of its own holding them ([Deep dive] §11, partial reuse)."""
    for s, d in zip(src_pages, dst_pages):
        pool[int(d)] = pool[int(s)]


def gather(pool, block_table_row, L: int, g: int, kv_dtype: str, k_scale=None, v_scale=None,
           start: int = 0):
    """K, V of tokens start..L-1 of one sequence and kv head g, as float64 [L-start][D]."""
    P = pool.shape[3]
    t = np.arange(start, L)
    pages = block_table_row[t // P]
    slots = t % P
    kb = pool[pages, 0, g, slots, :]
    vb = pool[pages, 1, g, slots, :]
    if kv_dtype == "fp8":
        return (decode_e4m3(kb) * np.float64(np.float32(k_scale[g])),
                decode_e4m3(vb) * np.float64(np.float32(v_scale[g])))
    if kv_dtype == "mxfp4":
        D = pool.shape[4] * 32 // 33
        return mx_decode(kb[:, :D], kb[:, D:]), mx_decode(vb[:, :D], vb[:, D:])
    return to_f64(kb, kv_dtype), to_f64(vb, kv_dtype)


def attend_rows(q_rows, K, V, scale, limits=None, return_weights=False, lower=None):
    """Softmax attention of query rows [R][D] over keys/values [L][D] in float64.

    Row r attends to keys lower[r] <= t < limits[r] (no bound where None).  Returns
    (out [R][D], lse [R]) and, on request, the weights [R][L]."""
    z = np.float64(scale) * (q_rows @ K.T)
    t = np.arange(K.shape[0])
    if limits is not None:
        z = np.where(t[None, :] < np.asarray(limits)[:, None], z, -np.inf)
    if lower is not None:
        z = np.where(t[None, :] >= np.asarray(lower)[:, None], z, -np.inf)
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    lsum = e.sum(axis=1)
    w = e / lsum[:, None]
    out = w @ V
    lse = m + np.log(lsum)
    if return_weights:
        return out, lse, w
    return out, lse


def window_start(pos: int, window: int) -> int:
    """First key a query at position `pos` attends to: 0, or with a limited attention
    window of W tokens the W newest positions up to and including its own, keys
    pos - W + 1 .. pos ([Deep dive] §11: tokens outside a sliding window take no
    further part in attention; the pages leave the boundary open and this is the
    plainest reading)."""
    return max(0, pos - window + 1) if window > 0 else 0


def decode(pool, block_tables, context_lens, q, q_dtype, sm_scale, kv_dtype,
           k_scale=None, v_scale=None, return_weights=False, window=0):
    """One decode step's attention: every query head of sequence s attends to all
    context_lens[s] tokens in the cache, the token appended this step included
    ([Deep dive] §2: a decode step reads the whole history; appending first means
    the new token attends to itself, as in causal attention) -- or, with a window W,
    to the last W of them.

    q is [S][Hq][D] in q_dtype; returns (out [S][Hq][D], lse [S][Hq]) float64."""
    S, Hq, D = q.shape
    Hkv = pool.shape[2]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D))
    lse = np.zeros((S, Hq))
    weights = {}
    for s in range(S):
        L = int(context_lens[s])
        lo = window_start(L - 1, window)
        for g in range(Hkv):
            K, V = gather(pool, block_tables[s], L, g, kv_dtype, k_scale, v_scale, start=lo)
            rows = to_f64(q[s, g * G:(g + 1) * G], q_dtype)
            res = attend_rows(rows, K, V, np.float32(sm_scale), None, return_weights)
            out[s, g * G:(g + 1) * G] = res[0]
            lse[s, g * G:(g + 1) * G] = res[1]
            if return_weights:
                weights[(s, g)] = res[2]
    if return_weights:
        return out, lse, weights
    return out, lse


def prefill_chunk(pool, block_tables, context_lens, cu_q_lens, q, q_dtype, sm_scale,
                  kv_dtype, k_scale=None, v_scale=None, window=0):
    """Causal attention of a prefill chunk against the cache it was just appended to.

    Sequence s has C = cu_q_lens[s+1] - cu_q_lens[s] query tokens; query i sits at
    position p = context_lens[s] - C + i and attends to keys 0..p ([Deep dive] §8:
    a long prompt is cut into chunks, each chunk adds its KV to the cache and later
    chunks continue from it) -- or, with a window W, to keys p - W + 1 .. p.  q is
    packed [total_q][Hq][D]; returns (out [total_q][Hq][D], lse [total_q][Hq])
    float64."""
    T, Hq, D = q.shape
    Hkv = pool.shape[2]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    lse = np.zeros((T, Hq))
    for s in range(len(context_lens)):
        a, b = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        C, L = b - a, int(context_lens[s])
        if C == 0:
            continue
        pos = L - C + np.arange(C)
        lo = window_start(int(pos[0]), window)     # keys before the first query's window
        limits = pos + 1 - lo                      # keys t < p_i + 1 (gathered from lo)
        lower = np.array([window_start(int(p), window) for p in pos]) - lo
        for g in range(Hkv):
            K, V = gather(pool, block_tables[s], L, g, kv_dtype, k_scale, v_scale, start=lo)
            rows = to_f64(q[a:b, g * G:(g + 1) * G], q_dtype).reshape(C * G, D)
            o, l = attend_rows(rows, K, V, np.float32(sm_scale), np.repeat(limits, G),
                               lower=np.repeat(lower, G))
            out[a:b, g * G:(g + 1) * G] = o.reshape(C, G, D)
            lse[a:b, g * G:(g + 1) * G] = l.reshape(C, G)
    return out, lse


def partition_stats(q_rows, K, V, scale, lo: int, hi: int):
    """Softmax statistics of query rows over the key partition [lo, hi):
    m = max z, l = sum exp(z - m), o = sum exp(z - m) V (not normalised).
    An empty partition gives m = -inf, l = 0, o = 0."""
    R, D = q_rows.shape
    if hi <= lo:
        return np.full(R, -np.inf), np.zeros(R), np.zeros((R, D))
    z = np.float64(scale) * (q_rows @ K[lo:hi].T)
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    return m, e.sum(axis=1), e @ V[lo:hi]


def lse_merge(parts):
    """Merge partition statistics [(m, l, o), ...] into (out, lse):
    M = max_j m_j, out = sum_j e^(m_j - M) o_j / sum_j e^(m_j - M) l_j,
    lse = M + ln sum_j e^(m_j - M) l_j.  Empty partitions (m = -inf) weigh 0."""
    ms = np.stack([p[0] for p in parts])
    M = ms.max(axis=0)
    wts = np.where(np.isfinite(ms), np.exp(ms - M[None, :]), 0.0)
    lsum = sum(w * p[1] for w, p in zip(wts, parts))
    osum = sum(w[:, None] * p[2] for w, p in zip(wts, parts))
    return osum / lsum[:, None], M + np.log(lsum)
