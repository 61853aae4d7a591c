"""Seeded synthetic inputs for attention over a paged KV cache.

This module is shared by the HIP path's tests/bench and by the CPU oracle's tests,
so it deliberately holds none of the method's arithmetic: no attention, no softmax,
no page-slot addressing and no FP8 encoding.  It describes one attention layer's
batch as

  * per-sequence lengths (``context_lens`` = tokens in the cache *after* this step's
    append, ``new_lens`` = tokens appended this step),
  * a block table per sequence (logical page i -> physical page id, -1 = unused),
  * logical per-token K/V values and packed query values, drawn from seeded
    streams and cast to the storage dtype (f32, or bf16 bit patterns as uint16),
  * fill constants for the page pool (NaN for pages no table names, a large finite
    poison for the slots of a named page that no token occupies).

How those tokens are laid out inside a page pool is up to each consumer.

Pages cited (by title):
  [Deep dive]  "NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践"
  [Concept]    "TensorRT-LLM" (concept explainer: 3 秒看懂 / 15 分钟专家深入)

The five workloads follow the pages' serving shapes: a decode step appends one
token per sequence and then reads the whole history ([Deep dive] §2, the
prefill/decode outline); the pool hands out fixed-size pages on growth through a
block table ([Deep dive] §9, the logical-block -> physical-block figure; [Concept]
关键机制, PagedAttention); mixed batches put context (prefill) requests before
generation requests ([Deep dive] §6); chunked prefill appends a chunk and then
attends causally ([Deep dive] §8); several requests may point at the same
physical prefix pages ([Deep dive] §10); the KV cache may be stored as FP8
([Deep dive] §13).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

BASE_SEED = 413

# Stream kinds for SeedSequence spawn keys.
_LENS, _PERM, _Q, _K, _V, _PK, _PV = range(7)

STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def _rng(cfg: int, kind: int, idx: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=BASE_SEED, spawn_key=(cfg, kind, idx))
    return np.random.Generator(np.random.PCG64(ss))


def _normal_f32(cfg: int, kind: int, idx: int, shape) -> np.ndarray:
    return _rng(cfg, kind, idx).standard_normal(size=shape, dtype=np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 values to a storage dtype: f32 as is, bf16 by round-to-nearest-even
    (bit patterns as uint16).  fp8 is not an input dtype (it is the cache's encoding)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"not an input dtype: {dtype}")


def fill_bits(kv_dtype: str):
    """(nan_fill, poison_fill) scalars of the storage dtype.

    NaN marks pages that no block table names; poison (3e4, or 448 for FP8) marks
    slots of a named page that no token occupies.  A kernel that reads either one
    produces a visibly wrong result."""
    if kv_dtype == "f32":
        return (np.array([0x7FC00000], np.uint32).view(np.float32)[0], np.float32(3.0e4))
    if kv_dtype == "bf16":
        return (np.uint16(0x7FC0), to_storage(np.array([3.0e4], np.float32), "bf16")[0])
    if kv_dtype == "fp8":
        return (np.uint8(0x7F), np.uint8(0x7E))
    if kv_dtype == "mxfp4":
        # bytes of codes and scales alike: 0xFF makes every scale NaN (E8M0 255);
        # 0x97 makes scales 2^24 and codes 6 / -0.5
        return (np.uint8(0xFF), np.uint8(0x97))
    raise ValueError(kv_dtype)


@dataclass
class Workload:
    """One attention layer's batch.  Sequences [0, num_prefill) are chunked-prefill
    requests (query chunk = their new tokens); the rest are decode sequences."""

    name: str
    cfg: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str
    q_dtype: str
    num_pages: int
    context_lens: np.ndarray          # int32 [S], after this step's append
    new_lens: np.ndarray              # int32 [S], appended this step
    block_tables: np.ndarray          # int32 [S][max_pages], -1 = unused
    num_prefill: int = 0
    num_splits: int = 0               # 0 = let the library choose
    window: int = 0                   # limited attention window in tokens (0 = none)
    prefix_len: int = 0               # shared-prefix tokens (0 = none)
    group_of: np.ndarray | None = None   # int32 [S], prefix group per sequence
    group_owner: np.ndarray | None = None  # int32 [groups], a member of each group
    _tok_cache: dict = field(default_factory=dict, repr=False)
    _scales: tuple | None = field(default=None, repr=False)

    # ---- shapes -------------------------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def sm_scale(self) -> np.float32:
        return np.float32(1.0 / math.sqrt(self.head_dim))

    @property
    def in_dtype(self) -> str:
        """dtype of the K/V values handed to kv_append (bf16 feeds an FP8 cache)."""
        return "f32" if self.kv_dtype == "f32" else "bf16"

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    def cu(self, lens: np.ndarray) -> np.ndarray:
        out = np.zeros(len(lens) + 1, np.int32)
        np.cumsum(lens, out=out[1:])
        return out

    def referenced_pages(self) -> np.ndarray:
        bt = self.block_tables
        return np.unique(bt[bt >= 0])

    def kv_bytes_logical(self) -> int:
        """K and V bytes of every attended token of the decode sequences, each read
        once per sequence (shared prefix pages counted once per sequence)."""
        L = self.context_lens[self.num_prefill:].astype(np.int64)
        n = int(L.sum()) * 2 * self.num_kv_heads * self.head_dim
        if self.kv_dtype == "mxfp4":       # half a byte per element + a scale byte per 32
            return n // 2 + n // 32
        return n * {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]

    # ---- values ---------------------------------------------------------------------
    def _private_start(self, s: int) -> int:
        if self.prefix_len and self.group_of is not None and self.group_of[s] >= 0:
            return self.prefix_len
        return 0

    def _seq_tokens(self, s: int):
        key = ("seq", s)
        if key not in self._tok_cache:
            lo, L = self._private_start(s), int(self.context_lens[s])
            shape = (L - lo, self.num_kv_heads, self.head_dim)
            k = _normal_f32(self.cfg, _K, s, shape)
            v = _normal_f32(self.cfg, _V, s, shape)
            self._tok_cache[key] = (to_storage(k, self.in_dtype), to_storage(v, self.in_dtype))
        return self._tok_cache[key]

    def _prefix_tokens(self, grp: int):
        key = ("grp", grp)
        if key not in self._tok_cache:
            shape = (self.prefix_len, self.num_kv_heads, self.head_dim)
            k = _normal_f32(self.cfg, _PK, grp, shape)
            v = _normal_f32(self.cfg, _PV, grp, shape)
            self._tok_cache[key] = (to_storage(k, self.in_dtype), to_storage(v, self.in_dtype))
        return self._tok_cache[key]

    def prefetch(self, seqs=None, threads: int | None = None):
        """Draw the per-sequence streams in parallel (NumPy's generators release the GIL)."""
        seqs = range(self.num_seqs) if seqs is None else seqs
        threads = threads or min(16, os.cpu_count() or 1)
        jobs = [("seq", s) for s in seqs]
        if self.prefix_len and self.group_owner is not None:
            jobs += [("grp", g) for g in range(len(self.group_owner))]
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda j: self._seq_tokens(j[1]) if j[0] == "seq" else self._prefix_tokens(j[1]), jobs))

    def drop_cache(self):
        self._tok_cache.clear()

    def tokens(self, s: int, lo: int = 0, hi: int | None = None):
        """(k, v) storage arrays [hi-lo][Hkv][D] for positions [lo, hi) of sequence s."""
        L = int(self.context_lens[s])
        hi = L if hi is None else hi
        assert 0 <= lo <= hi <= L
        p0 = self._private_start(s)
        parts_k, parts_v = [], []
        if lo < p0:
            pk, pv = self._prefix_tokens(int(self.group_of[s]))
            parts_k.append(pk[lo:min(hi, p0)])
            parts_v.append(pv[lo:min(hi, p0)])
        if hi > p0:
            k, v = self._seq_tokens(s)
            a = max(lo, p0) - p0
            parts_k.append(k[a:hi - p0])
            parts_v.append(v[a:hi - p0])
        if len(parts_k) == 1:
            return parts_k[0], parts_v[0]
        shape = (0, self.num_kv_heads, self.head_dim)
        if not parts_k:
            z = np.zeros(shape, STORAGE[self.in_dtype])
            return z, z.copy()
        return np.concatenate(parts_k), np.concatenate(parts_v)

    def q_packed(self) -> np.ndarray:
        """Queries, packed [sum(new_lens)][Hq][D] in sequence order (prefill first)."""
        n = int(self.new_lens.sum())
        q = _normal_f32(self.cfg, _Q, 0, (n, self.num_q_heads, self.head_dim))
        return to_storage(q, self.q_dtype)

    def step_kv(self):
        """K/V appended this step, packed [sum(new_lens)][Hkv][D] in sequence order."""
        ks, vs = [], []
        for s in range(self.num_seqs):
            L, n = int(self.context_lens[s]), int(self.new_lens[s])
            k, v = self.tokens(s, L - n, L)
            ks.append(k)
            vs.append(v)
        return np.concatenate(ks), np.concatenate(vs)

    def history_plan(self):
        """Appends that bring the cache to its state before this step.

        Yields (rows, context_lens_after, new_lens, k_packed, v_packed): `rows` index
        the sequences (and block-table rows) the append covers.  The shared prefix of
        each group is written once, through the group owner's table; every sequence
        then appends its private history."""
        if self.prefix_len and self.group_owner is not None:
            rows = self.group_owner.astype(np.int32)
            ks, vs = zip(*[self._prefix_tokens(g) for g in range(len(rows))])
            yield (rows, np.full(len(rows), self.prefix_len, np.int32),
                   np.full(len(rows), self.prefix_len, np.int32),
                   np.concatenate(ks), np.concatenate(vs))
        rows, ctx, new, ks, vs = [], [], [], [], []
        for s in range(self.num_seqs):
            lo, hi = self._private_start(s), int(self.context_lens[s] - self.new_lens[s])
            if hi <= lo:
                continue
            k, v = self.tokens(s, lo, hi)
            rows.append(s)
            ctx.append(hi)
            new.append(hi - lo)
            ks.append(k)
            vs.append(v)
        if rows:
            yield (np.array(rows, np.int32), np.array(ctx, np.int32), np.array(new, np.int32),
                   np.concatenate(ks), np.concatenate(vs))

    # ---- FP8 calibration ------------------------------------------------------------
    def fp8_scales(self):
        """(k_scale, v_scale, k_inv_scale, v_inv_scale), float32 [Hkv] each.

        Per-(layer, kv-head) calibration on the synthetic data ([Concept] 关键机制,
        quantization: scales are calibrated when the engine is built): scale = amax/448
        over that head's K (resp. V) values of every token in the batch, computed in
        float64 and rounded to float32; the quantizing multiplier is f32(1/f64(scale))."""
        if self._scales is None:
            amax_k = np.zeros(self.num_kv_heads)
            amax_v = np.zeros(self.num_kv_heads)

            def upd(kv):
                for arr, amax in ((kv[0], amax_k), (kv[1], amax_v)):
                    a = _storage_to_f32(arr, self.in_dtype)
                    np.maximum(amax, np.abs(a).max(axis=(0, 2)), out=amax)

            for s in range(self.num_seqs):
                upd(self._seq_tokens(s))
            if self.prefix_len and self.group_owner is not None:
                for g in range(len(self.group_owner)):
                    upd(self._prefix_tokens(g))
            ks = (amax_k / 448.0).astype(np.float32)
            vs = (amax_v / 448.0).astype(np.float32)
            kinv = (1.0 / ks.astype(np.float64)).astype(np.float32)
            vinv = (1.0 / vs.astype(np.float64)).astype(np.float32)
            self._scales = (ks, vs, kinv, vinv)
        return self._scales


def _storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return a
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float().numpy()


# ---- block-table construction --------------------------------------------------------

def _assign_pages(cfg: int, pages_per_seq, num_pages: int, shared=None):
    """Hand out physical pages in seeded-permutation order, sequence by sequence.

    `shared` = (group_of, prefix_pages, groups): the first `prefix_pages` logical pages
    of every member of a group point at the group's pages, handed out first."""
    perm = _rng(cfg, _PERM).permutation(num_pages).astype(np.int32)
    S = len(pages_per_seq)
    max_pages = int(max(pages_per_seq)) if S else 1
    bt = np.full((S, max(max_pages, 1)), -1, np.int32)
    nxt = 0
    if shared is not None:
        group_of, npre, groups = shared
        gp = []
        for _ in range(groups):
            gp.append(perm[nxt:nxt + npre])
            nxt += npre
        for s in range(S):
            bt[s, :npre] = gp[group_of[s]]
    for s in range(S):
        lo = shared[1] if shared is not None else 0
        n = int(pages_per_seq[s]) - lo
        bt[s, lo:lo + n] = perm[nxt:nxt + n]
        nxt += n
    assert nxt <= num_pages
    return bt


def _cdiv(a, b):
    return -(-a // b)


def make(cfg: int, **over) -> Workload:
    """Build workload `cfg` (1..6).  Keyword overrides shrink it for fast tests:
    num_seqs, len_range, num_prefill, prefill_chunk, prefill_cached, context_len,
    prefix_len, group_size, num_splits, tokens; `window` (any workload) limits every
    query's attention to the W newest positions up to its own."""
    builders = {1: _cfg1, 2: _cfg2, 3: _cfg3, 4: _cfg4, 5: _cfg5, 6: _cfg6}
    window = int(over.pop("window", 0))
    wl = builders[cfg](**over)
    wl.window = window
    return wl


def _cfg6(**o):
    """Multi-token decode (the speculative-verification shape), bf16: the Llama-3-8B
    batch of workload 2 -- 64 sequences, context lengths U[512,4096] counting this
    step's tokens, 32/8 heads, D=128, page 64 -- with `tokens` (4) new tokens per
    sequence appended and attended causally as prefill chunks in one call.  Overrides:
    num_seqs, len_range, tokens."""
    S = o.get("num_seqs", 64)
    lo, hi = o.get("len_range", (512, 4096))
    T = o.get("tokens", 4)
    L = _uniform_lens(6, S, lo, hi)
    P = 64
    pps = _cdiv(L, P)
    npages = _pool_for(pps)
    bt = _assign_pages(6, pps, npages)
    return Workload("spec_verify4_bf16" if T == 4 else f"spec_verify{T}_bf16", 6, 32, 8, 128, P, "bf16",
                    "bf16", npages, L, np.full_like(L, T), bt, num_prefill=S, num_splits=0)


def _cfg1(**o):
    """Tiny paged decode, fp32: 4 sequences of lengths {17,64,100,250}, 8/8 heads,
    D=64, page 16, a pool of 64 pages handed out by seeded permutation."""
    L = np.array(o.get("lens", [17, 64, 100, 250]), np.int32)
    P = o.get("page_size", 16)
    npages = o.get("num_pages", 64)
    pps = _cdiv(L, P)
    bt = _assign_pages(1, pps, npages)
    return Workload("tiny_fp32_decode", 1, 8, 8, 64, P, "f32", "f32", npages, L,
                    np.ones_like(L), bt, num_splits=o.get("num_splits", 0))


def _uniform_lens(cfg, S, lo, hi):
    return _rng(cfg, _LENS).integers(lo, hi + 1, size=S).astype(np.int32)


def _pool_for(pps, shared_pages=0):
    return int(math.ceil(1.25 * (int(np.sum(pps)) + shared_pages)))


def _cfg2(**o):
    """Llama-3-8B-shaped decode, bf16: 64 sequences, lengths U[512,4096], 32/8 heads,
    D=128, page 64, pool 1.25x the pages needed.  Overrides for small test variants:
    num_seqs, len_range or explicit lens, page_size, num_q_heads, num_kv_heads,
    head_dim, num_splits, kv_dtype ("mxfp4": an OCP MXFP4 cache)."""
    if "lens" in o:
        L = np.array(o["lens"], np.int32)
    else:
        S = o.get("num_seqs", 64)
        lo, hi = o.get("len_range", (512, 4096))
        L = _uniform_lens(2, S, lo, hi)
    P = o.get("page_size", 64)
    pps = _cdiv(L, P)
    npages = _pool_for(pps)
    bt = _assign_pages(2, pps, npages)
    kv = o.get("kv_dtype", "bf16")
    return Workload(f"llama3_8b_decode_{kv}", 2, o.get("num_q_heads", 32), o.get("num_kv_heads", 8),
                    o.get("head_dim", 128), P, kv, "bf16", npages, L, np.ones_like(L), bt,
                    num_splits=o.get("num_splits", 0))


def _cfg3(**o):
    """Mixed in-flight batch, bf16: 2 chunked-prefill requests (512-token chunk against
    8192 cached tokens) packed first, then 256 decode sequences with lognormal lengths
    (median 1024, sigma 1.0, clipped to [16,16384]); 32/8 heads, D=128, page 64.
    Overrides for test variants: num_seqs, num_prefill, prefill_chunk and
    prefill_cached (scalars or one per prefill request), median, clip, page_size,
    num_q_heads, num_kv_heads, head_dim, num_splits, kv_dtype ("fp8": an E4M3 cache,
    "mxfp4": an OCP MXFP4 cache)."""
    S = o.get("num_seqs", 256)
    npf = o.get("num_prefill", 2)
    C = np.broadcast_to(np.asarray(o.get("prefill_chunk", 512), np.int32), (npf,))
    cached = np.broadcast_to(np.asarray(o.get("prefill_cached", 8192), np.int32), (npf,))
    clip = o.get("clip", (16, 16384))
    med = o.get("median", 1024)
    z = _rng(3, _LENS).standard_normal(S)
    Ld = np.clip(np.rint(np.exp(math.log(med) + 1.0 * z)), clip[0], clip[1]).astype(np.int32)
    L = np.concatenate([(cached + C).astype(np.int32), Ld])
    new = np.concatenate([C.astype(np.int32), np.ones(S, np.int32)])
    P = o.get("page_size", 64)
    pps = _cdiv(L, P)
    npages = _pool_for(pps)
    bt = _assign_pages(3, pps, npages)
    kv = o.get("kv_dtype", "bf16")
    return Workload("mixed_inflight_bf16" if kv == "bf16" else f"mixed_inflight_{kv}", 3,
                    o.get("num_q_heads", 32), o.get("num_kv_heads", 8), o.get("head_dim", 128), P, kv,
                    "bf16", npages, L, new, bt, num_prefill=npf, num_splits=o.get("num_splits", 0))


def _cfg4(**o):
    """Long-context split-KV decode, bf16: 8 sequences of 131072 tokens, 32/8 heads,
    D=128, page 128, 64 page-aligned partitions per sequence."""
    S = o.get("num_seqs", 8)
    Lc = o.get("context_len", 131072)
    L = np.full(S, Lc, np.int32)
    P = 128
    pps = _cdiv(L, P)
    npages = _pool_for(pps)
    bt = _assign_pages(4, pps, npages)
    return Workload("long_context_splitkv_bf16", 4, 32, 8, 128, P, "bf16", "bf16", npages, L,
                    np.ones_like(L), bt, num_splits=o.get("num_splits", 64))


def _cfg5(**o):
    """FP8-E4M3 KV cache with a shared prefix: 128 decode sequences, 64/8 heads, D=128,
    page 64, lengths U[2049,8192]; groups of 32 consecutive requests share the physical
    pages of a 2048-token prefix."""
    S = o.get("num_seqs", 128)
    gs = o.get("group_size", 32)
    pre = o.get("prefix_len", 2048)
    lo, hi = o.get("len_range", (pre + 1, 8192))
    P = 64
    assert pre % P == 0 and S % gs == 0 and lo > pre
    L = _uniform_lens(5, S, lo, hi)
    groups = S // gs
    group_of = (np.arange(S) // gs).astype(np.int32)
    pps = _cdiv(L, P)
    npre = pre // P
    npages = _pool_for(pps - npre, groups * npre)
    bt = _assign_pages(5, pps, npages, shared=(group_of, npre, groups))
    owner = (np.arange(groups) * gs).astype(np.int32)
    return Workload("fp8_shared_prefix_decode", 5, 64, 8, 128, P, "fp8", "bf16", npages, L,
                    np.ones_like(L), bt, num_splits=o.get("num_splits", 0), prefix_len=pre,
                    group_of=group_of, group_owner=owner)
