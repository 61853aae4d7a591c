/*
 * paged_kv.h -- C ABI of libpagedkv.so: attention over a paged KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title):
 *   [Deep dive]  "NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践"
 *   [Concept]    "TensorRT-LLM" (concept explainer)
 *
 * The KV cache of one attention layer is a pool of fixed-size pages; a sequence's
 * block table maps its logical page i to a physical page, and pages are handed out
 * as the sequence grows ([Deep dive] §9, the logical-block -> physical-block
 * figure; [Concept] 关键机制, PagedAttention).  The page size is a power of two
 * greater than 1 ([Deep dive] §9, the block-pool facts).  Each engine step hands
 * the kernels the positions and page tables of the batch ([Concept] 技术原理,
 * 运行时执行模型, step 2), packed without padding, context (prefill) requests
 * before generation requests ([Deep dive] §6).
 *
 * Conventions for every entry point
 *   - Pointers named in a struct or argument are DEVICE pointers unless marked
 *     HOST.  The caller owns every buffer; the library never allocates, frees or
 *     synchronizes.  Buffers must stay alive until the stream passes the launch.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call only enqueues work on it and returns.
 *   - Return value: PKV_OK (0) or a negative pkv_status_t.  Every precondition the
 *     host can check is checked before anything is launched; on error nothing is
 *     enqueued and paged_kv_last_error() describes the problem.
 *   - Values the host cannot see (page ids inside a block table, device-side
 *     lengths) must satisfy the stated contract; a violation is undefined
 *     behaviour (typically a memory fault), exactly as an out-of-range index into
 *     any device array -- unless PKV_DEBUG=1 is set in the environment: then every
 *     call first validates them on the device (reading only the block tables,
 *     lengths and prefix sums, or the page pairs of a copy), and a call that breaks
 *     the contract touches neither the pool nor its outputs and raises bits that
 *     paged_kv_debug_status() reports.  The variable is read at every call.
 *   - Calls are reentrant: the library keeps no state but cached device
 *     properties, a thread-local error string, a thread-local test override
 *     (paged_kv_debug_set_auto_waves) and, per device, the validation flag words.
 */
#ifndef PAGED_KV_H
#define PAGED_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_F32 = 0,       /* IEEE binary32 */
  PKV_BF16 = 1,      /* bfloat16 */
  PKV_FP8_E4M3 = 2,  /* OCP FP8 E4M3 ("fn": bias 7, max 448, S.1111.111 = NaN) */
  PKV_MXFP4 = 3      /* OCP MXFP4: E2M1 elements, one E8M0 scale per 32 (cache only) */
} pkv_dtype_t;

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* a null pointer, a bad size or an inconsistent argument */
  PKV_EUNSUPPORTED = -2,  /* a valid combination the library has no kernel for */
  PKV_EWORKSPACE = -3,    /* workspace missing or smaller than the size function says */
  PKV_ELAUNCH = -4        /* the HIP runtime refused the launch */
} pkv_status_t;

/* One layer's page pool.
 *   pool: [num_pages][2][num_kv_heads][tile] elements of cache_dtype, one tile of
 *         page_size * head_dim elements per (page, K|V, kv head); index 0 of the
 *         second axis is K, 1 is V.  A page holds the K and V of page_size
 *         consecutive tokens of one sequence.  16-byte aligned.
 *           K tile: [head_dim / 32][page_size][32]: 32-dim chunks, token-major
 *                   inside a chunk (32 dims of one token are contiguous)
 *           V tile: [page_size / S][head_dim][S] with S = min(page_size, 32): dim-major
 *                   inside sub-blocks of S slots (a dim's S tokens are contiguous);
 *                   with S = 32, slot r of a sub-block sits at position
 *                   8 * ((r mod 16) div 4) + 4 * (r div 16) + (r mod 4)
 *         Both are the operand layouts of the matrix cores, so that every 64-lane
 *         load is one contiguous kilobyte; one 32-token block's V is one run.
 *         A page, [2][num_kv_heads][tile], is one contiguous range of the pool.
 *         MXFP4 tiles (paged_kv_page_bytes gives the page size in bytes) hold
 *         page_size * head_dim / 2 bytes of E2M1 codes, two per byte (the element
 *         listed first in the low nibble), then page_size * head_dim / 32 E8M0
 *         scale bytes, one per 32 consecutive dims of a token row:
 *           K codes:  one row of head_dim / 2 bytes per slot; inside a row, dims
 *                     32j + 8c .. 32j + 8c + 7 are the 4 bytes at 4 * (c * head_dim
 *                     / 32 + j), c = 0..3
 *           K scales: [page_size][head_dim / 32]
 *           V codes:  32-slot sub-blocks of 16 * head_dim bytes; in a sub-block the
 *                     codes of dim 16u + m at positions 8c .. 8c + 7 (positions as
 *                     in the V tile above) are the 4 bytes at 4 * ((4m + c) *
 *                     head_dim / 16 + u)
 *           V scales: [page_size / 32][32 positions][head_dim / 32]
 *   page_size: power of two, >= 2 (>= 32 for MXFP4).     head_dim: 64 or 128.
 *   k_scale / v_scale: FP8 only, [num_kv_heads] float32 dequantization
 *         multipliers (value = decoded code * scale); NULL for F32/BF16 caches.
 *   k_inv_scale / v_inv_scale: FP8 only, [num_kv_heads] float32 quantization
 *         multipliers used by kv_append (code = e4m3(f32(x * inv_scale)));
 *         NULL for F32/BF16 caches.
 * FP8 caches hold one scale per (layer, kv head) for K and for V ([Deep dive]
 * §13, KvCacheConfig(dtype="fp8"); [Concept] 关键机制, 量化方案: FP8 data is
 * widened back to 16 bits before accumulation). */
typedef struct pkv_cache {
  void* pool;
  int64_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t cache_dtype; /* pkv_dtype_t */
  const float* k_scale;
  const float* v_scale;
  const float* k_inv_scale;
  const float* v_inv_scale;
} pkv_cache_t;

/* The sequences of one call.
 *   block_tables: [num_seqs][max_pages_per_seq] int32, physical page of each
 *         logical page; entries past a sequence's last page are ignored (-1 by
 *         convention).  Every entry a call reads must lie in [0, num_pages).
 *   context_lens: [num_seqs] int32, tokens in the cache AFTER this step's append,
 *         1 <= context_lens[s] <= max_context_len.
 *   max_context_len: HOST value, an upper bound of context_lens used to size the
 *         grid; must satisfy max_context_len <= max_pages_per_seq * page_size.
 *   window: 0 = full attention; W > 0 = limited attention window: a query at
 *         position p attends to keys max(0, p - W + 1) .. p only ([Deep dive] §11,
 *         limited attention window: tokens outside a sliding window take no further
 *         part in attention, and their blocks can be released).  Block-table entries
 *         of pages that end at or before 32 * floor(lo / 32), lo = the first key the
 *         call's earliest query of the sequence sees, are never read (the caller may
 *         have released them: -1 or any value).  Ignored by kv_append and
 *         paged_kv_debug_gather. */
typedef struct pkv_seqs {
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t max_pages_per_seq;
  int32_t max_context_len;
  int32_t window; /* >= 0 */
} pkv_seqs_t;

/* Bytes of one page ([2][num_kv_heads][tile]) of a pool with these parameters, for
 * sizing pools: page_size * head_dim * 2 * num_kv_heads times the element size (4,
 * 2 or 1 bytes; 17/32 of a byte for MXFP4, scales included).  0 for parameters
 * pkv_cache_t does not allow. */
size_t paged_kv_page_bytes(int32_t cache_dtype, int32_t page_size, int32_t num_kv_heads,
                           int32_t head_dim);

/* kv_append -- write this step's new K/V rows into the slots the block tables name
 * ([Deep dive] §2: a decode step writes the new token's KV; §8: each prefill
 * chunk adds its KV to the cache; [Concept] 技术原理, 调度策略嵌入: the page-table
 * lookup in front of every KV read and write).
 *   k_new, v_new: packed [total_new][num_kv_heads][head_dim]; F32 for an F32
 *         cache, BF16 for BF16, FP8 and MXFP4 caches.
 *   cu_new_lens: [num_seqs + 1] int32 prefix sums (cu[0] = 0, cu[num_seqs] =
 *         total_new); sequence s writes rows cu[s] .. cu[s+1]-1 to positions
 *         context_lens[s] - n_s .. context_lens[s] - 1, n_s = cu[s+1] - cu[s].
 *   total_new: HOST value, rows in k_new / v_new (0 is a no-op).
 * Position t of sequence s lands in page block_tables[s][t / page_size], slot
 * t % page_size.  F32 and BF16 rows are copied bit for bit; an FP8 cache stores
 * e4m3(f32(x * inv_scale[head])) rounded to nearest-even and saturated to +-448.
 * An MXFP4 cache encodes every 32 consecutive dims of a row as one block (OCP MX
 * conversion): scale 2^(floor(log2 max|x|) - 2), clamped to [2^-127, 2^127] (2^-127
 * for a block of zeros); elements x / scale rounded to nearest-even on the E2M1
 * grid, magnitudes above 6 clamped to 6, sign bit from x.  Inputs must be finite.
 * Two rows of one call must not name the same slot. */
int kv_append(const pkv_cache_t* cache, const pkv_seqs_t* seqs, const void* k_new,
              const void* v_new, const int32_t* cu_new_lens, int32_t total_new,
              void* stream);

/* kv_copy_pages -- copy whole pages of the pool: page dst_pages[i] <- page
 * src_pages[i], K and V of every kv head, for i < num_pairs.  For copy-on-partial-
 * reuse ([Deep dive] §11, partial reuse: when a new request matches only the first
 * tokens of a cached block, those tokens are copied into a new block of its own, so
 * that several requests can reuse one block partly).  The destination's slots past
 * the matched tokens hold the source's later tokens; the new sequence's kv_append
 * overwrites them before any attention call reads them (attention reads only slots
 * below a sequence's length).
 *   src_pages, dst_pages: [num_pairs] int32 page ids in [0, num_pages); a destination
 *         page must not be a source page of the same call nor appear twice.
 *   num_pairs: HOST value, 0 .. 65535 (0 is a no-op).
 * Pool pages must be 16-byte multiples (always true for the supported sizes). */
int kv_copy_pages(const pkv_cache_t* cache, const int32_t* src_pages, const int32_t* dst_pages,
                  int32_t num_pairs, void* stream);

/* Workspace bytes paged_attn_decode needs for these arguments (0 when the call
 * runs as one partition per sequence).  Same argument rules as the call; 0 is also
 * returned for arguments the call would reject. */
size_t paged_attn_decode_workspace_size(const pkv_cache_t* cache, const pkv_seqs_t* seqs,
                                        int32_t q_dtype, int32_t num_q_heads,
                                        int32_t num_splits);

/* paged_attn_decode -- one generation step: each query head of sequence s attends
 * to all context_lens[s] cached tokens, the one appended this step included
 * ([Deep dive] §2: decode reads the whole KV history each step).
 *   q: [num_seqs][num_q_heads][head_dim] of q_dtype (F32 or BF16; BF16 only with an
 *         MXFP4 cache, whose values are decoded to bf16 exactly: code x 2^(E-127)).
 *   num_q_heads: a multiple of num_kv_heads; query head h reads kv head
 *         h / (num_q_heads / num_kv_heads).
 *   sm_scale: logit scale (1/sqrt(head_dim) in the usual model).
 *   num_splits: 0 = the library partitions the keys itself: with a BF16 or FP8
 *         cache, BF16 queries and pages of >= 8 tokens, or an MXFP4 cache, BF16
 *         queries and pages of >= 32 tokens (the matrix-core kernels)
 *         the 32-token blocks of all (sequence, kv head) pairs, each pair
 *         counting a few blocks more for its start, are cut into equal contiguous
 *         shares, one per wave that fits on the device at once;
 *         otherwise page-aligned partitions of at least 256 keys.  N > 0 = split
 *         each sequence's keys into page-aligned partitions of ceil(max_context_len
 *         / N) keys, rounded up to a page (and to 32 keys on the matrix-core
 *         path).  Partial results are merged by log-sum-exp (exact up to rounding).
 *   out: [num_seqs][num_q_heads][head_dim] of q_dtype.
 *   lse_out: NULL or [num_seqs][num_q_heads] float32, natural-log sum of exp of
 *         the scaled logits.
 *   workspace: device buffer of at least paged_attn_decode_workspace_size()
 *         bytes, 256-byte aligned (NULL allowed when that size is 0); its contents
 *         need no initialisation.  Calls that run at the same time must not share
 *         a workspace.
 * Results depend only on logical positions: permuting physical pages (and the
 * tables with them) gives bit-identical output. */
int paged_attn_decode(const pkv_cache_t* cache, const pkv_seqs_t* seqs, const void* q,
                      int32_t q_dtype, int32_t num_q_heads, float sm_scale,
                      int32_t num_splits, void* out, float* lse_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* paged_attn_decode_noalloc -- paged_attn_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same call without a workspace argument.  Its workspace is
 * a device array the library owns, PKV_NOALLOC_SCRATCH_BYTES per device, held from
 * the moment the library is loaded on a device until the process ends; the call
 * allocates nothing.  Same arguments, kernels and results as paged_attn_decode (bit
 * for bit).  PKV_EWORKSPACE when the call's plan needs more than the array holds
 * (paged_attn_decode_workspace_size gives the need: about 4.2 MB for a 64-sequence,
 * 32/8-head, head_dim 128 decode batch; 8.5 MB for 8 sequences in 64 fixed
 * partitions).  Every call on one device shares that device's array, and the array
 * keeps the last call's partial results: calls that overlap in time on one device
 * (several streams, or several host threads) race and must not be issued. */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
int paged_attn_decode_noalloc(const pkv_cache_t* cache, const pkv_seqs_t* seqs, const void* q,
                              int32_t q_dtype, int32_t num_q_heads, float sm_scale,
                              int32_t num_splits, void* out, float* lse_out, void* stream);

/* paged_attn_prefill_chunk -- causal attention of prompt chunks against the cache
 * the chunks were just appended to ([Deep dive] §8, chunked prefill: every chunk
 * but the last is a multiple of the block size; §6: context requests are packed
 * first).  Query i of sequence s sits at position context_lens[s] - C_s + i and
 * attends to keys 0 .. that position.
 *   q: packed [total_q][num_q_heads][head_dim] of q_dtype (F32 or BF16; BF16 with a
 *         BF16 or FP8 cache and pages of >= 8 tokens, or an MXFP4 cache and pages of
 *         >= 32 tokens, runs on the matrix cores; there,
 *         chunks of at most 16 / G queries -- several tokens verified per sequence,
 *         as in speculative decoding -- run on the balanced decode kernels, all
 *         queries of a (sequence, kv head) sharing one pass over its keys).
 *   cu_q_lens: [num_seqs + 1] int32 prefix sums of the chunk lengths C_s, with
 *         C_s <= context_lens[s].
 *   total_q, max_q_len: HOST values (rows of q; an upper bound of C_s).
 *   out: [total_q][num_q_heads][head_dim] of q_dtype; lse_out: NULL or
 *         [total_q][num_q_heads] float32.
 *   workspace: device buffer of at least paged_attn_prefill_workspace_size() bytes,
 *         256-byte aligned (NULL allowed when that size is 0); no initialisation
 *         needed; not shared by calls that run at the same time. */
/* Workspace bytes paged_attn_prefill_chunk needs for these arguments (0 when none;
 * also 0 for arguments the call would reject).  total_q and max_q_len are HOST
 * values as in the call. */
size_t paged_attn_prefill_workspace_size(const pkv_cache_t* cache, const pkv_seqs_t* seqs,
                                         int32_t q_dtype, int32_t num_q_heads, int32_t total_q,
                                         int32_t max_q_len);

int paged_attn_prefill_chunk(const pkv_cache_t* cache, const pkv_seqs_t* seqs,
                             const void* q, int32_t q_dtype, const int32_t* cu_q_lens,
                             int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                             float sm_scale, void* out, float* lse_out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* paged_kv_debug_gather -- copy every cached token back into logical order, for
 * checking the pool's contents bit for bit.  Uses the page-slot addressing of
 * kv_append (and of the vector-ALU attention kernels); the matrix-core kernels'
 * own loaders are checked by paged_kv_debug_gather_operands.
 *   k_out, v_out: [num_seqs][max_context_len][num_kv_heads][head_dim] of
 *         cache_dtype; rows t >= context_lens[s] are left untouched.  For MXFP4 a
 *         row is head_dim / 2 bytes of codes in dim order (two per byte, the lower
 *         dim in the low nibble) then its head_dim / 32 scale bytes. */
int paged_kv_debug_gather(const pkv_cache_t* cache, const pkv_seqs_t* seqs, void* k_out,
                          void* v_out, void* stream);

/* paged_kv_debug_gather_operands -- run the matrix-core attention kernels' own page
 * loaders over every cached token and write the K and V operands they produce back in
 * logical order, for checking the hot path's page-gather indexing bit for bit
 * ([Deep dive] §9, the logical-block -> physical-block figure).
 *   path: 0 = the decode loaders (a 32-token block straight from the pool into
 *         operand registers, page ids from a register window of the table; pages of
 *         8 or 16 tokens look each token's page up); 1 = the prefill loaders (a block
 *         fetched by a whole workgroup, decoded and staged in LDS, then read back with
 *         the operand lane map; pages of >= 32 tokens); 2 = the loaders of the dense FP8
 *         decode kernel (one-query FP8 calls with more (sequence, kv head) pairs than
 *         resident waves: raw FP8 blocks in flight, widened when folded; pages of >= 32).
 *   k_out, v_out: [num_seqs][max_context_len][num_kv_heads][head_dim] bfloat16: the
 *         values the products use -- bf16 caches as stored, FP8 codes widened exactly
 *         (the per-head scale is applied to the products, not to the operands), MXFP4
 *         elements times their block scale (exact).  Rows t >= context_lens[s] are
 *         left untouched.
 * Caches: BF16 or FP8 with pages of >= 8 tokens (path 1: >= 32), MXFP4 (pages >= 32),
 * path 2 FP8 only (pages >= 32); PKV_EUNSUPPORTED otherwise. */
int paged_kv_debug_gather_operands(const pkv_cache_t* cache, const pkv_seqs_t* seqs, int32_t path,
                                   void* k_out, void* v_out, void* stream);

/* paged_kv_stream_read -- measurement helper: read `bytes` of a device buffer once, at
 * the decode kernels' launch shape (one 64-lane wave per SIMD, 16-byte non-temporal loads,
 * eight 1 KiB loads in flight per wave), and write one word per wave to `sink`.  Its rate
 * is the practical HBM-read ceiling the attention kernels are compared with.
 *   src: 1024-byte aligned; bytes: a multiple of 1024.
 *   sink: device buffer of paged_kv_stream_read_waves() 32-bit words (contents meaningless). */
int paged_kv_stream_read(const void* src, size_t bytes, void* sink, void* stream);
/* Waves (and sink words) of paged_kv_stream_read on the current device (<= 16384). */
int32_t paged_kv_stream_read_waves(void);

/* Contract violations found by device validation (PKV_DEBUG=1), as bits. */
typedef enum {
  PKV_DEBUG_PAGE_RANGE = 1,  /* a page id the call addresses is outside [0, num_pages) */
  PKV_DEBUG_LENGTH = 2,      /* a length outside [1, max_context_len], n_s > L_s, or a
                                prefill chunk longer than L_s or max_q_len */
  PKV_DEBUG_CU = 4,          /* prefix sums not starting at 0, decreasing, or not ending
                                at total_new / total_q */
  PKV_DEBUG_DUP_SLOT = 8,    /* two appended rows name the same (page, slot) */
  PKV_DEBUG_COPY_PAIRS = 16  /* a copy destination that is also a source, or repeated */
} pkv_debug_flag_t;

/* The pkv_debug_flag_t bits raised by validated calls on the current device since the
 * last clear (0 = none), then cleared if `clear` is nonzero; negative pkv_status_t on
 * error.  Waits for the whole device to finish its work (a debugging call, not for
 * a hot loop).  Validated calls share the device's flag words: validated calls on
 * several streams at once race on them. */
int32_t paged_kv_debug_status(int32_t clear);

/* Test-only: make the balanced decode schedule use `waves` waves instead of the
 * device's resident count (0 restores it), for the calls of the calling thread --
 * few waves give long shares and many cut segments on small batches.  The workspace
 * size query and the call must see the same setting. */
int paged_kv_debug_set_auto_waves(int32_t waves);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* paged_kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */
