// C-ABI front end of libpagedkv: argument validation, partition choice and dispatch.
// Every host-checkable precondition is checked here, before anything is launched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/paged_kv.h"
#include "device_common.h"
#include "internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return PKV_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int ilog2_exact(int v) {
  if (v < 2 || (v & (v - 1))) return -1;
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute-unit count of the current device, cached per device.
int cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (dev >= int(cache.size())) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace

namespace pkv {
// The error reporting of the front end, for entry points defined in other sources.
int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int resident_blocks(const void* kernel, int block) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  auto key = std::make_pair(dev, kernel);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  const int r = per_cu * n;
  cache[key] = r;
  return r;
}
}  // namespace pkv

namespace {

int check_cache(const pkv_cache_t* c, pkv::CacheArgs& out) {
  if (!c) return fail(PKV_EINVAL, "cache is NULL");
  if (!c->pool) return fail(PKV_EINVAL, "cache->pool is NULL");
  if (!aligned(c->pool, 16)) return fail(PKV_EINVAL, "cache->pool must be 16-byte aligned");
  if (c->num_pages < 1) return fail(PKV_EINVAL, "cache->num_pages must be >= 1 (got %lld)", (long long)c->num_pages);
  const int lp = ilog2_exact(c->page_size);
  if (lp < 0 || c->page_size > 4096)
    return fail(PKV_EINVAL, "cache->page_size must be a power of two in [2, 4096] (got %d)", c->page_size);
  if (c->num_kv_heads < 1) return fail(PKV_EINVAL, "cache->num_kv_heads must be >= 1");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "cache->head_dim must be 64 or 128 (got %d)", c->head_dim);
  if (c->cache_dtype != PKV_F32 && c->cache_dtype != PKV_BF16 && c->cache_dtype != PKV_FP8_E4M3 &&
      c->cache_dtype != PKV_MXFP4)
    return fail(PKV_EINVAL, "cache->cache_dtype %d is not a pkv_dtype_t", c->cache_dtype);
  if (c->cache_dtype == PKV_MXFP4 && c->page_size < 32)
    return fail(PKV_EUNSUPPORTED, "an MXFP4 cache needs pages of >= 32 tokens (got %d)", c->page_size);
  out.pool = c->pool;
  out.num_pages = c->num_pages;
  out.page_size = c->page_size;
  out.log2_page = lp;
  out.num_kv_heads = c->num_kv_heads;
  out.head_dim = c->head_dim;
  out.dtype = c->cache_dtype;
  out.k_scale = c->k_scale;
  out.v_scale = c->v_scale;
  out.k_inv_scale = c->k_inv_scale;
  out.v_inv_scale = c->v_inv_scale;
  out.debug_flag = nullptr;
  return PKV_OK;
}

int check_seqs(const pkv_seqs_t* s, const pkv::CacheArgs& c, pkv::SeqArgs& out) {
  if (!s) return fail(PKV_EINVAL, "seqs is NULL");
  if (s->window < 0) return fail(PKV_EINVAL, "seqs->window must be >= 0");
  if (s->num_seqs < 0) return fail(PKV_EINVAL, "seqs->num_seqs must be >= 0");
  out.window = s->window;
  out.num_seqs = s->num_seqs;
  out.block_tables = s->block_tables;
  out.context_lens = s->context_lens;
  out.max_pages_per_seq = s->max_pages_per_seq;
  out.max_context_len = s->max_context_len;
  if (s->num_seqs == 0) return PKV_OK;
  if (!s->block_tables) return fail(PKV_EINVAL, "seqs->block_tables is NULL");
  if (!s->context_lens) return fail(PKV_EINVAL, "seqs->context_lens is NULL");
  if (s->max_pages_per_seq < 1) return fail(PKV_EINVAL, "seqs->max_pages_per_seq must be >= 1");
  if (s->max_context_len < 1) return fail(PKV_EINVAL, "seqs->max_context_len must be >= 1");
  if (int64_t(s->max_context_len) > int64_t(s->max_pages_per_seq) * c.page_size)
    return fail(PKV_EINVAL, "seqs->max_context_len (%d) exceeds max_pages_per_seq * page_size (%lld)",
                s->max_context_len, (long long)s->max_pages_per_seq * c.page_size);
  return PKV_OK;
}

int check_fp8_scales(const pkv::CacheArgs& c, bool inv) {
  if (c.dtype != PKV_FP8_E4M3) return PKV_OK;
  if (inv ? (!c.k_inv_scale || !c.v_inv_scale) : (!c.k_scale || !c.v_scale))
    return fail(PKV_EINVAL, "an FP8 cache needs %s", inv ? "k_inv_scale and v_inv_scale" : "k_scale and v_scale");
  return PKV_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

struct DecodePlan {
  bool mfma;       // matrix-core kernels (else the vector-ALU kernel)
  bool auto_mode;  // matrix-core balanced schedule
  bool dense;      // auto, FP8: the two-waves-per-SIMD kernel (more segments than waves)
  int waves;       // auto: workgroups launched
  int chunk, max_splits;
  size_t off_desc, off_lse, off_o, ws_bytes;
};

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

constexpr int kMinShareBlocks = 4;  // auto schedule: at least 4 x 32 tokens per wave

// Test-only override of the balanced schedule's wave count (paged_kv_debug_set_auto_waves;
// 0 = the device's resident count).  Thread-local, like the error string: it changes only
// the calls the setting thread makes, and nothing but that explicit call sets it.
thread_local int g_auto_waves_override = 0;

// Waves of the balanced schedule: the device's resident count of the chosen kernel, or
// the test override.
int auto_waves(int kv_dtype, int head_dim, int group, int page_size, bool dense = false) {
  if (g_auto_waves_override > 0) return g_auto_waves_override;
  return std::max(1, pkv::mfma_auto_waves(kv_dtype, head_dim, group, page_size, dense));
}

// Device validation of a call before its kernels, when PKV_DEBUG=1 is set in the
// environment (read at every call; validation adds one small launch per call).
bool debug_mode() {
  const char* e = std::getenv("PKV_DEBUG");
  return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

int validate(pkv::CacheArgs& c, const pkv::SeqArgs& s, const pkv::ValidateArgs& v, hipStream_t st) {
  if (!debug_mode()) return PKV_OK;
  const hipError_t e = pkv::launch_validate(c, s, v, st);
  if (e != hipSuccess) return fail(PKV_ELAUNCH, "device validation: launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

// Partition plan of one decode call.
//  * Matrix-core path (bf16 / FP8 caches, bf16 queries, pages >= 8 tokens):
//    num_splits == 0 spreads all (sequence, kv head, 32-token block) work evenly over
//    the waves that fit on the device at once; num_splits == N > 0 cuts every
//    sequence into page-aligned partitions of ceil(max_context_len / N) tokens
//    (rounded up to a page and to 32 tokens), one wave each.
//  * Vector-ALU path: N > 0 as above (page-aligned); 0 aims at a few work items per
//    compute unit, never below 256 keys per partition.
// Workspace: partial log-sum-exps and normalised partial outputs (fp32), after one
// 16-byte descriptor per wave for the balanced schedule.
DecodePlan plan_decode(const pkv::CacheArgs& c, const pkv::SeqArgs& s, int num_q_heads,
                       int q_dtype, int num_splits, int record_rows = 0) {
  const int P = c.page_size;
  const int64_t maxL = s.max_context_len;
  const int G = num_q_heads / c.num_kv_heads;
  DecodePlan p{};
  p.mfma = pkv::mfma_decode_supported(c.dtype, q_dtype, c.head_dim, G, P);
  if (p.mfma && num_splits == 0) {
    p.auto_mode = true;
    p.waves = auto_waves(c.dtype, c.head_dim, G, P);
    // One query per sequence, FP8, pages of >= 32 tokens: more (sequence, kv head)
    // segments than waves take the dense kernel (its own resident count)
    if (record_rows == 0 && c.dtype == pkv::DT_FP8 && P >= 32 && int64_t(s.num_seqs) * c.num_kv_heads > p.waves) {
      p.dense = true;
      p.waves = auto_waves(c.dtype, c.head_dim, G, P, true);
    }
    p.chunk = 0;
    p.max_splits = 0;
    const size_t recs = size_t(2) * p.waves;  // up to two cut segments per wave
    const size_t rows = record_rows > 0 ? size_t(record_rows) : size_t(G);  // tile rows per record
    p.off_desc = 0;
    p.off_lse = align256(size_t(p.waves) * 16);
    p.off_o = p.off_lse + align256(recs * rows * sizeof(float));
    p.ws_bytes = p.off_o + align256(recs * rows * c.head_dim * sizeof(float));
    return p;
  }
  int64_t chunk;
  if (num_splits > 0) {
    const int64_t gran = p.mfma ? std::max(P, 32) : P;
    chunk = cdiv(cdiv(maxL, num_splits), gran) * gran;
    chunk = std::min<int64_t>(chunk, cdiv(maxL, gran) * gran);
  } else {
    const int64_t target = 8LL * cu_count();
    const int64_t est = cdiv(int64_t(s.num_seqs) * c.num_kv_heads * maxL, target);
    chunk = cdiv(std::max<int64_t>(est, std::max(256, P)), P) * P;
    chunk = std::min<int64_t>(std::max<int64_t>(chunk, P), cdiv(maxL, P) * P);
  }
  p.chunk = int(chunk);
  p.max_splits = int(cdiv(maxL, chunk));
  if (p.max_splits <= 1) {
    p.max_splits = 1;
    p.ws_bytes = 0;
    return p;
  }
  const size_t slots = size_t(s.num_seqs) * num_q_heads * p.max_splits;  // (row, q head, split)
  p.off_desc = 0;
  p.off_lse = 0;
  p.off_o = align256(slots * sizeof(float));
  p.ws_bytes = p.off_o + align256(slots * c.head_dim * sizeof(float));
  return p;
}

// Prefill plan.  Matrix-core path: work items (a workgroup sharing one K/V stream, or
// a single wave for pages shorter than 32 tokens) of a fixed number of queries of one
// (sequence, kv head); when those do not fill the device's resident work items, each
// item's key range is cut into equal splits (at most 16, each >= 8 blocks of 32 keys
// on average), merged afterwards.  Workspace: per (query row, kv head, split) the
// partial log-sum-exps (G floats) and normalised outputs (G x D floats).
struct PrefillPlan {
  bool mfma;
  int qtiles, splits;
  size_t off_lse, off_o, ws_bytes;
  // Chunks of at most 16 / G queries (speculative-verification and similar short
  // chunks): all queries of a (sequence, kv head) fit one 16-row MFMA tile, so the call
  // runs on the balanced decode kernels -- HBM-bound streaming of each sequence's K/V
  // once -- instead of the query-tiled prefill kernels.
  bool via_decode;
  DecodePlan dec;
  int per_wave;  // chunks the per-wave prefill kernel runs (see mfma_prefill_geometry)
};

PrefillPlan plan_prefill(const pkv::CacheArgs& c, const pkv::SeqArgs& s, int num_q_heads,
                         int q_dtype, int total_q, int max_q_len) {
  PrefillPlan p{};
  const int G = num_q_heads / c.num_kv_heads;
  p.mfma = pkv::mfma_decode_supported(c.dtype, q_dtype, c.head_dim, G, c.page_size);
  if (!p.mfma) return p;
  if (G <= 8 && int64_t(max_q_len) * G <= 16) {
    p.dec = plan_decode(c, s, num_q_heads, q_dtype, 0, 16);
    if (p.dec.auto_mode) {
      p.via_decode = true;
      p.ws_bytes = p.dec.ws_bytes;
      return p;
    }
  }
  int qw = 1, resident_items = 1;
  pkv::mfma_prefill_geometry(c.dtype, c.head_dim, G, c.page_size, max_q_len, &qw, &resident_items, &p.per_wave);
  p.qtiles = int(cdiv(max_q_len, qw));
  const int64_t base = int64_t(s.num_seqs) * c.num_kv_heads * p.qtiles;
  const int64_t resident = std::max(1, resident_items);
  int64_t splits = std::max<int64_t>(1, resident / std::max<int64_t>(base, 1));
  splits = std::min<int64_t>(splits, 16);
  const int64_t span = s.window > 0 ? std::min<int64_t>(s.max_context_len, int64_t(s.window) + max_q_len)
                                    : s.max_context_len;  // keys one query group sees at most
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, cdiv(span, 32) / 8));
  p.splits = int(splits);
  if (p.splits == 1) return p;
  const size_t recs = size_t(total_q) * c.num_kv_heads * p.splits;
  p.off_lse = 0;
  p.off_o = align256(recs * G * sizeof(float));
  p.ws_bytes = p.off_o + align256(recs * G * c.head_dim * sizeof(float));
  return p;
}

int check_attn(const pkv::CacheArgs& c, int q_dtype, int num_q_heads, bool /*decode*/) {
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16)
    return fail(PKV_EINVAL, "q_dtype must be PKV_F32 or PKV_BF16 (got %d)", q_dtype);
  if (num_q_heads < 1 || num_q_heads % c.num_kv_heads)
    return fail(PKV_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, c.num_kv_heads);
  const int G = num_q_heads / c.num_kv_heads;
  if (!pkv::valu_supported(c.dtype, q_dtype, c.head_dim, G) &&
      !pkv::mfma_decode_supported(c.dtype, q_dtype, c.head_dim, G, c.page_size))
    return fail(PKV_EUNSUPPORTED, "no kernel for cache dtype %d, q dtype %d, head_dim %d, group %d",
                c.dtype, q_dtype, c.head_dim, G);
  return check_fp8_scales(c, false);
}

}  // namespace

extern "C" {

const char* paged_kv_last_error(void) { return g_error.c_str(); }

size_t paged_kv_page_bytes(int32_t cache_dtype, int32_t page_size, int32_t num_kv_heads, int32_t head_dim) {
  pkv_cache_t c{};
  c.pool = reinterpret_cast<void*>(uintptr_t(256));  // a placeholder: only the sizes are checked
  c.num_pages = 1;
  c.page_size = page_size;
  c.num_kv_heads = num_kv_heads;
  c.head_dim = head_dim;
  c.cache_dtype = cache_dtype;
  pkv::CacheArgs a;
  if (check_cache(&c, a) != PKV_OK) return 0;
  ok();
  return size_t(2) * num_kv_heads * size_t(pkv::tile_bytes(cache_dtype, page_size, head_dim));
}

int kv_append(const pkv_cache_t* cache, const pkv_seqs_t* seqs, const void* k_new,
              const void* v_new, const int32_t* cu_new_lens, int32_t total_new, void* stream) {
  pkv::CacheArgs c;
  pkv::SeqArgs s;
  int st;
  if ((st = check_cache(cache, c)) != PKV_OK) return st;
  if ((st = check_seqs(seqs, c, s)) != PKV_OK) return st;
  if (total_new < 0) return fail(PKV_EINVAL, "total_new must be >= 0");
  if (total_new == 0 || s.num_seqs == 0) return ok();
  if (!k_new || !v_new || !cu_new_lens) return fail(PKV_EINVAL, "k_new, v_new and cu_new_lens must not be NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(PKV_EINVAL, "k_new and v_new must be 16-byte aligned");
  if ((st = check_fp8_scales(c, true)) != PKV_OK) return st;
  const int in_dtype = c.dtype == PKV_F32 ? PKV_F32 : PKV_BF16;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = validate(c, s, pkv::ValidateArgs{pkv::VK_APPEND, cu_new_lens, total_new, 0, nullptr, nullptr, 0}, hs)) != PKV_OK)
    return st;
  return launch_status(pkv::launch_kv_append(c, s, k_new, v_new, in_dtype, cu_new_lens, total_new, hs),
                       "kv_append");
}

int kv_copy_pages(const pkv_cache_t* cache, const int32_t* src_pages, const int32_t* dst_pages,
                  int32_t num_pairs, void* stream) {
  pkv::CacheArgs c;
  int st;
  if ((st = check_cache(cache, c)) != PKV_OK) return st;
  if (num_pairs < 0) return fail(PKV_EINVAL, "num_pairs must be >= 0");
  if (num_pairs > 65535) return fail(PKV_EINVAL, "num_pairs must be <= 65535 per call");
  if (num_pairs == 0) return ok();
  if (!src_pages || !dst_pages) return fail(PKV_EINVAL, "src_pages and dst_pages must not be NULL");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  pkv::SeqArgs none{};
  if ((st = validate(c, none, pkv::ValidateArgs{pkv::VK_COPY, nullptr, 0, 0, src_pages, dst_pages, num_pairs}, hs)) !=
      PKV_OK)
    return st;
  return launch_status(pkv::launch_copy_pages(c, src_pages, dst_pages, num_pairs, hs), "kv_copy_pages");
}

size_t paged_attn_decode_workspace_size(const pkv_cache_t* cache, const pkv_seqs_t* seqs,
                                        int32_t q_dtype, int32_t num_q_heads, int32_t num_splits) {
  pkv::CacheArgs c;
  pkv::SeqArgs s;
  if (check_cache(cache, c) != PKV_OK || check_seqs(seqs, c, s) != PKV_OK) return 0;
  if (s.num_seqs == 0 || num_splits < 0) return 0;
  if (check_attn(c, q_dtype, num_q_heads, true) != PKV_OK) return 0;
  return plan_decode(c, s, num_q_heads, q_dtype, num_splits).ws_bytes;
}

int paged_attn_decode(const pkv_cache_t* cache, const pkv_seqs_t* seqs, const void* q,
                      int32_t q_dtype, int32_t num_q_heads, float sm_scale, int32_t num_splits,
                      void* out, float* lse_out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  pkv::AttnArgs a{};
  int st;
  if ((st = check_cache(cache, a.cache)) != PKV_OK) return st;
  if ((st = check_seqs(seqs, a.cache, a.seqs)) != PKV_OK) return st;
  if ((st = check_attn(a.cache, q_dtype, num_q_heads, true)) != PKV_OK) return st;
  if (num_splits < 0) return fail(PKV_EINVAL, "num_splits must be >= 0");
  if (a.seqs.num_seqs == 0) return ok();
  if (!q || !out) return fail(PKV_EINVAL, "q and out must not be NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(PKV_EINVAL, "q and out must be 16-byte aligned");
  const DecodePlan p = plan_decode(a.cache, a.seqs, num_q_heads, q_dtype, num_splits);
  if (p.ws_bytes) {
    if (!workspace || workspace_bytes < p.ws_bytes)
      return fail(PKV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                  workspace ? workspace_bytes : size_t(0));
    if (!aligned(workspace, 256)) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
  }
  char* ws = static_cast<char*>(workspace);
  a.q = q;
  a.q_dtype = q_dtype;
  a.num_q_heads = num_q_heads;
  a.sm_scale = sm_scale;
  a.out = out;
  a.lse_out = lse_out;
  a.chunk = p.chunk;
  a.max_splits = p.max_splits;
  a.ws_lse = p.ws_bytes ? reinterpret_cast<float*>(ws + p.off_lse) : nullptr;
  a.ws_o = p.ws_bytes ? reinterpret_cast<float*>(ws + p.off_o) : nullptr;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = validate(a.cache, a.seqs, pkv::ValidateArgs{pkv::VK_DECODE, nullptr, 0, 0, nullptr, nullptr, 0}, hs)) !=
      PKV_OK)
    return st;
  if (p.mfma) {
    a.num_waves = p.waves;
    a.min_share = kMinShareBlocks;
    a.ws_desc = p.auto_mode ? reinterpret_cast<int4*>(ws + p.off_desc) : nullptr;
    pkv::MfmaPlan mp{p.auto_mode, p.waves, false, p.dense};
    return launch_status(pkv::launch_mfma_decode(a, mp, hs), "paged_attn_decode");
  }
  return launch_status(pkv::launch_valu_decode(a, hs), "paged_attn_decode");
}

size_t paged_attn_prefill_workspace_size(const pkv_cache_t* cache, const pkv_seqs_t* seqs,
                                         int32_t q_dtype, int32_t num_q_heads, int32_t total_q,
                                         int32_t max_q_len) {
  pkv::CacheArgs c;
  pkv::SeqArgs s;
  if (check_cache(cache, c) != PKV_OK || check_seqs(seqs, c, s) != PKV_OK) return 0;
  if (s.num_seqs == 0 || total_q <= 0 || max_q_len <= 0) return 0;
  if (check_attn(c, q_dtype, num_q_heads, false) != PKV_OK) return 0;
  return plan_prefill(c, s, num_q_heads, q_dtype, total_q, max_q_len).ws_bytes;
}

int paged_attn_prefill_chunk(const pkv_cache_t* cache, const pkv_seqs_t* seqs, const void* q,
                             int32_t q_dtype, const int32_t* cu_q_lens, int32_t total_q,
                             int32_t max_q_len, int32_t num_q_heads, float sm_scale, void* out,
                             float* lse_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  pkv::AttnArgs a{};
  int st;
  if ((st = check_cache(cache, a.cache)) != PKV_OK) return st;
  if ((st = check_seqs(seqs, a.cache, a.seqs)) != PKV_OK) return st;
  if ((st = check_attn(a.cache, q_dtype, num_q_heads, false)) != PKV_OK) return st;
  if (total_q < 0 || max_q_len < 0) return fail(PKV_EINVAL, "total_q and max_q_len must be >= 0");
  if (a.seqs.num_seqs == 0 || total_q == 0) return ok();
  if (!q || !out || !cu_q_lens) return fail(PKV_EINVAL, "q, out and cu_q_lens must not be NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(PKV_EINVAL, "q and out must be 16-byte aligned");
  if (max_q_len < 1 || max_q_len > a.seqs.max_context_len)
    return fail(PKV_EINVAL, "max_q_len (%d) must be in [1, max_context_len]", max_q_len);
  const PrefillPlan p = plan_prefill(a.cache, a.seqs, num_q_heads, q_dtype, total_q, max_q_len);
  if (p.ws_bytes) {
    if (!workspace || workspace_bytes < p.ws_bytes)
      return fail(PKV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                  workspace ? workspace_bytes : size_t(0));
    if (!aligned(workspace, 256)) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
  }
  a.q = q;
  a.q_dtype = q_dtype;
  a.num_q_heads = num_q_heads;
  a.sm_scale = sm_scale;
  a.out = out;
  a.lse_out = lse_out;
  a.cu_q_lens = cu_q_lens;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = validate(a.cache, a.seqs,
                     pkv::ValidateArgs{pkv::VK_PREFILL, cu_q_lens, total_q, max_q_len, nullptr, nullptr, 0}, hs)) !=
      PKV_OK)
    return st;
  if (p.via_decode) {
    char* ws = static_cast<char*>(workspace);
    a.ws_lse = reinterpret_cast<float*>(ws + p.dec.off_lse);
    a.ws_o = reinterpret_cast<float*>(ws + p.dec.off_o);
    a.ws_desc = reinterpret_cast<int4*>(ws + p.dec.off_desc);
    a.num_waves = p.dec.waves;
    a.min_share = kMinShareBlocks;
    pkv::MfmaPlan mp{true, p.dec.waves, true, false};
    return launch_status(pkv::launch_mfma_decode(a, mp, hs), "paged_attn_prefill_chunk");
  }
  if (p.mfma) {
    char* ws = static_cast<char*>(workspace);
    a.max_splits = p.splits;
    a.pf_qtiles = p.qtiles;
    a.pf_per_wave = p.per_wave;
    a.ws_lse = p.ws_bytes ? reinterpret_cast<float*>(ws + p.off_lse) : nullptr;
    a.ws_o = p.ws_bytes ? reinterpret_cast<float*>(ws + p.off_o) : nullptr;
    return launch_status(pkv::launch_mfma_prefill(a, hs), "paged_attn_prefill_chunk");
  }
  a.chunk = int(cdiv(a.seqs.max_context_len, a.cache.page_size) * a.cache.page_size);
  a.max_splits = 1;
  return launch_status(pkv::launch_valu_prefill(a, hs), "paged_attn_prefill_chunk");
}

int paged_kv_debug_gather(const pkv_cache_t* cache, const pkv_seqs_t* seqs, void* k_out,
                          void* v_out, void* stream) {
  pkv::CacheArgs c;
  pkv::SeqArgs s;
  int st;
  if ((st = check_cache(cache, c)) != PKV_OK) return st;
  if ((st = check_seqs(seqs, c, s)) != PKV_OK) return st;
  if (s.num_seqs == 0) return ok();
  if (s.num_seqs > 65535) return fail(PKV_EUNSUPPORTED, "debug gather handles at most 65535 sequences");
  if (!k_out || !v_out) return fail(PKV_EINVAL, "k_out and v_out must not be NULL");
  if (!aligned(k_out, 16) || !aligned(v_out, 16)) return fail(PKV_EINVAL, "k_out and v_out must be 16-byte aligned");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = validate(c, s, pkv::ValidateArgs{pkv::VK_GATHER, nullptr, 0, 0, nullptr, nullptr, 0}, hs)) != PKV_OK)
    return st;
  return launch_status(pkv::launch_debug_gather(c, s, k_out, v_out, hs), "paged_kv_debug_gather");
}

int paged_kv_debug_gather_operands(const pkv_cache_t* cache, const pkv_seqs_t* seqs, int32_t path,
                                   void* k_out, void* v_out, void* stream) {
  pkv::CacheArgs c;
  pkv::SeqArgs s;
  int st;
  if ((st = check_cache(cache, c)) != PKV_OK) return st;
  if ((st = check_seqs(seqs, c, s)) != PKV_OK) return st;
  if (path < 0 || path > 2)
    return fail(PKV_EINVAL, "path must be 0 (decode loaders), 1 (prefill loaders) or 2 (dense FP8 decode loaders)");
  if (!pkv::operands_supported(c.dtype, c.page_size, c.head_dim, path))
    return fail(PKV_EUNSUPPORTED, "no matrix-core loader for cache dtype %d, page size %d, path %d", c.dtype,
                c.page_size, path);
  if (s.num_seqs == 0) return ok();
  if (int64_t(s.num_seqs) * c.num_kv_heads > (int64_t(1) << 31) - 1)
    return fail(PKV_EUNSUPPORTED, "too many (sequence, kv head) pairs");
  if (!k_out || !v_out) return fail(PKV_EINVAL, "k_out and v_out must not be NULL");
  if (!aligned(k_out, 16) || !aligned(v_out, 16)) return fail(PKV_EINVAL, "k_out and v_out must be 16-byte aligned");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = validate(c, s, pkv::ValidateArgs{pkv::VK_GATHER, nullptr, 0, 0, nullptr, nullptr, 0}, hs)) != PKV_OK)
    return st;
  return launch_status(pkv::launch_debug_operands(c, s, path, k_out, v_out, hs), "paged_kv_debug_gather_operands");
}

// One wave per SIMD (four per compute unit), as the decode kernels run.
int32_t paged_kv_stream_read_waves(void) {
  ok();
  return std::min(4 * cu_count(), 1 << 14);
}

int paged_kv_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return fail(PKV_EINVAL, "src and sink must not be NULL");
  if (!aligned(src, 1024) || bytes % 1024) return fail(PKV_EINVAL, "src must be 1024-byte aligned and bytes a multiple of 1024");
  if (!aligned(sink, 4)) return fail(PKV_EINVAL, "sink must be 4-byte aligned");
  if (bytes == 0) return ok();
  return launch_status(pkv::launch_stream_read(src, int64_t(bytes), static_cast<uint32_t*>(sink),
                                               std::min(4 * cu_count(), 1 << 14),
                                               static_cast<hipStream_t>(stream)),
                       "paged_kv_stream_read");
}

int32_t paged_kv_debug_status(int32_t clear) {
  int32_t bits = 0;
  const hipError_t e = pkv::read_debug_status(clear != 0, &bits);
  if (e != hipSuccess) return fail(PKV_ELAUNCH, "paged_kv_debug_status: %s", hipGetErrorString(e));
  ok();
  return bits;
}

int paged_kv_debug_set_auto_waves(int32_t waves) {
  if (waves < 0 || waves > (1 << 16)) return fail(PKV_EINVAL, "waves must be in [0, 65536] (got %d)", waves);
  g_auto_waves_override = waves;
  return ok();
}

}  // extern "C"
