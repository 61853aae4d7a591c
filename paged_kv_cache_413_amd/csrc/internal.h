// Internal launch interface between the C-ABI front end (api.cpp) and the kernel
// translation units.  Arguments are validated by the front end before any launcher
// is called; launchers only enqueue work and return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct CacheArgs {
  void* pool;
  int64_t num_pages;
  int page_size, log2_page, num_kv_heads, head_dim, dtype;
  const float *k_scale, *v_scale, *k_inv_scale, *v_inv_scale;
  // Device validation (PKV_DEBUG=1): the word the call's validation kernel writes; every
  // kernel of the call returns at once when it is nonzero.  NULL when not validating.
  const int32_t* debug_flag;
};

// True when the call's device validation found a contract violation: the kernel must
// return before touching the pool or any output (every thread of a workgroup sees the
// same word, so a workgroup with barriers leaves as a whole).
__device__ __forceinline__ bool halted(const CacheArgs& c) { return c.debug_flag && *c.debug_flag != 0; }

struct SeqArgs {
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs, max_pages_per_seq, max_context_len;
  int window;  // 0 = full attention, else keys p - window + 1 .. p of a query at p
};

// kv_append
hipError_t launch_kv_append(const CacheArgs& c, const SeqArgs& s, const void* k_new,
                            const void* v_new, int in_dtype, const int32_t* cu_new_lens,
                            int total_new, hipStream_t stream);

// Attention.  Rows are decode sequences (cu_q_lens == nullptr: row r = sequence r,
// keys 0..context_lens[r]-1) or packed prefill queries (row r = query i of the
// sequence s with cu_q_lens[s] <= r < cu_q_lens[s+1]; keys 0..L_s - C_s + i).
struct AttnArgs {
  CacheArgs cache;
  SeqArgs seqs;
  const void* q;
  int q_dtype, num_q_heads;
  float sm_scale;
  void* out;
  float* lse_out;
  const int32_t* cu_q_lens;  // prefill only
  int total_q, max_q_len;    // prefill only
  // split-KV (decode): partitions of `chunk` tokens (a multiple of the page size)
  int chunk, max_splits;
  float* ws_o;    // normalised partial outputs (layout per kernel family)
  float* ws_lse;  // partial log-sum-exp
  // matrix-core decode, auto schedule: resident waves, minimum blocks per wave and the
  // per-wave descriptor of its first (sequence, kv head) segment
  int num_waves, min_share;
  int4* ws_desc;
  // matrix-core prefill: query tiles per (sequence, kv head) (key splits: max_splits),
  // and whether the per-wave kernel runs them (else the LDS-shared one)
  int pf_qtiles;
  int pf_per_wave;
};

// Occupancy-derived number of workgroups of `block` threads of `kernel` that fit on
// the current device at once (cached per device and kernel).
int resident_blocks(const void* kernel, int block);

// General vector-ALU kernels (attn_valu.hip): every supported combination.
bool valu_supported(int kv_dtype, int q_dtype, int head_dim, int group);
hipError_t launch_valu_decode(const AttnArgs& a, hipStream_t stream);
hipError_t launch_valu_prefill(const AttnArgs& a, hipStream_t stream);

// Matrix-core decode kernels (attn_mfma.hip): bf16 / FP8 caches with bf16 queries,
// page sizes >= 8, groups of up to 16 query heads per kv head.
struct MfmaPlan {
  bool auto_mode;    // true: balanced shares over `waves`; false: fixed partitions
  int waves;
  bool multi_query;  // auto only: several queries per sequence (prefill chunks of at most
                     // 16 / G queries, packed by cu_q_lens), 16-row partial records
  bool dense;        // auto, one query, FP8, pages >= 32: the two-waves-per-SIMD kernel
};
bool mfma_decode_supported(int kv_dtype, int q_dtype, int head_dim, int group, int page_size);
int mfma_auto_waves(int kv_dtype, int head_dim, int group, int page_size, bool dense = false);
hipError_t launch_mfma_decode(const AttnArgs& a, const MfmaPlan& p, hipStream_t stream);

// Matrix-core prefill kernels (prefill_mfma.hip): same support as the decode kernels.
// Queries of one (sequence, kv head) per work item and work items resident at once,
// for the prefill kernel these arguments select.
void mfma_prefill_geometry(int kv_dtype, int head_dim, int group, int page_size, int max_q_len,
                           int* queries_per_item, int* resident_items, int* per_wave);
hipError_t launch_mfma_prefill(const AttnArgs& a, hipStream_t stream);

// Device validation of one call (validate.hip), launched before its kernels when
// PKV_DEBUG=1: page ids the call addresses in [0, num_pages), lengths within their
// bounds, consistent prefix sums, no two appended rows in one slot, valid copy pairs.
// On success c.debug_flag points at the word the kernels check.
enum ValidateKind : int { VK_APPEND = 0, VK_DECODE = 1, VK_PREFILL = 2, VK_GATHER = 3, VK_COPY = 4 };
struct ValidateArgs {
  int kind;
  const int32_t* cu;   // append: cu_new_lens; prefill: cu_q_lens; else NULL
  int total_rows;      // append: total_new; prefill: total_q
  int max_q_len;       // prefill
  const int32_t *src, *dst;  // copy pairs
  int num_pairs;
};
hipError_t launch_validate(CacheArgs& c, const SeqArgs& s, const ValidateArgs& v, hipStream_t stream);
// Sticky violation bits of the current device since the last clear (synchronizes the device).
hipError_t read_debug_status(bool clear, int32_t* out);

// Page copy and debug gather
hipError_t launch_copy_pages(const CacheArgs& c, const int32_t* src, const int32_t* dst, int n,
                             hipStream_t stream);
hipError_t launch_debug_gather(const CacheArgs& c, const SeqArgs& s, void* k_out, void* v_out,
                               hipStream_t stream);

// Plain streaming read (stream_read.hip), one wave per workgroup.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int waves, hipStream_t stream);

// The attention kernels' own loaders over every cached token (debug_gather.hip): path 0
// the decode block pipeline, path 1 the prefill kernel's LDS staging; bf16 operands out.
bool operands_supported(int kv_dtype, int page_size, int head_dim, int path);
hipError_t launch_debug_operands(const CacheArgs& c, const SeqArgs& s, int path, void* k_out, void* v_out,
                                 hipStream_t stream);

}  // namespace pkv
