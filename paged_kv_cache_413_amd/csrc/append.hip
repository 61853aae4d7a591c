// kv_append and the debug gather: moving token rows between packed logical order and
// their slots in the page pool.
//
// A decode step writes the new token's K/V into the cache and a prefill chunk writes
// its whole chunk ("NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践", §2 and
// §8); the slot comes from the block-table lookup that sits in front of every KV
// read and write ("TensorRT-LLM", 技术原理, 调度策略嵌入).
//
// One workgroup per packed row; each thread moves 8 consecutive elements of one
// (K|V, head) row, so a bf16 row of 8 heads x 128 dims is 256 threads x 16 bytes read.
// K rows are stored with one vector store; V goes to the dim-major V tile, one
// element per dim.  MXFP4 caches have kernels of their own below (block encoding).
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace pkv {
namespace {

// Sequence that owns packed row `row`: the largest s with cu[s] <= row.  cu is
// non-decreasing from cu[0] = 0, so that is the number of s in 1 .. num_seqs-1 with
// cu[s] <= row.  The lanes of a wave test 256 entries per round, all loads issued
// before any count: one memory round trip per round where a binary search takes
// log2(num_seqs) dependent ones.  The result is the same in every lane.
__device__ __forceinline__ int owner_of(const int32_t* __restrict__ cu, int num_seqs, int row) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  for (int b = 1; b < num_seqs; b += 256) {
    int v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = cu[min(b + 64 * k + lane, num_seqs - 1)];  // unconditional loads
    bool le[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) le[k] = b + 64 * k + lane < num_seqs && v[k] <= row;
#pragma unroll
    for (int k = 0; k < 4; ++k) cnt += __popcll(__ballot(le[k]));
  }
  return __builtin_amdgcn_readfirstlane(cnt);
}

// The 16 (bf16 or fp8 caches: bf16 in) or 32 (f32) input bytes one thread of the
// append moves.
template <int IN>
struct AppendSrc {
  uint4 w[IN == DT_F32 ? 2 : 1];
};

template <int IN>
__device__ __forceinline__ AppendSrc<IN> append_src(const void* __restrict__ in, int64_t elem) {
  AppendSrc<IN> r;
  if constexpr (IN == DT_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(in) + elem);
    r.w[0] = p[0];
    r.w[1] = p[1];
  } else {
    r.w[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + elem);
  }
  return r;
}

template <int IN, int KV>
__global__ __launch_bounds__(256) void kv_append_kernel(CacheArgs c, SeqArgs sq,
                                                        const void* __restrict__ k_new,
                                                        const void* __restrict__ v_new,
                                                        const int32_t* __restrict__ cu) {
  if (halted(c)) return;
  const int row = blockIdx.x;
  const int D = c.head_dim, H = c.num_kv_heads;
  const int vec_per_head = D / 8;
  const int vec_per_row = H * vec_per_head;
  const int log2P = c.log2_page;
  // Input element of item i; the first item's bytes are loaded before the slot lookup
  // (they depend on the row alone), so their latency overlaps its dependent loads.
  auto src_of = [&](int i, int& kv, int& h, int& e0) {
    kv = i >= vec_per_row;
    const int j = i - kv * vec_per_row;
    h = j / vec_per_head;
    e0 = (j - h * vec_per_head) * 8;
    return (int64_t(row) * H + h) * D + e0;
  };
  const int i0 = threadIdx.x;
  AppendSrc<IN> first{};
  if (i0 < 2 * vec_per_row) {
    int kv, h, e0;
    const int64_t src = src_of(i0, kv, h, e0);
    first = append_src<IN>(kv ? v_new : k_new, src);
  }
  const int s = owner_of(cu, sq.num_seqs, row);
  const int n = cu[s + 1] - cu[s];
  const int pos = sq.context_lens[s] - n + (row - cu[s]);
  const int32_t* bt = sq.block_tables + int64_t(s) * sq.max_pages_per_seq;
  for (int i = i0; i < 2 * vec_per_row; i += blockDim.x) {
    int kv, h, e0;
    const int64_t src = src_of(i, kv, h, e0);
    const AppendSrc<IN> in = i == i0 ? first : append_src<IN>(kv ? v_new : k_new, src);
    // K rows are contiguous in the tile (one vector store); V is dim-major inside its
    // sub-block, so the eight elements go to eight consecutive dims, one sub-block
    // length apart.
    const int64_t dst = elem_offset(bt, pos, log2P, kv, h, H, D, e0);
    const int64_t step = kv ? (int64_t(1) << v_sub_log2(log2P)) : 1;
    if constexpr (KV == DT_F32) {
      float* pool = static_cast<float*>(c.pool);
      if (!kv) {
        uint4* d4 = reinterpret_cast<uint4*>(pool + dst);
        d4[0] = in.w[0];
        d4[1] = in.w[1];
      } else {
        const uint4 a = in.w[0], b = in.w[1];
        const uint32_t x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) pool[dst + e * step] = __uint_as_float(x[e]);
      }
    } else if constexpr (KV == DT_BF16) {
      const uint4 w = in.w[0];
      uint16_t* pool = static_cast<uint16_t*>(c.pool);
      if (!kv) {
        *reinterpret_cast<uint4*>(pool + dst) = w;
      } else {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) pool[dst + e * step] = uint16_t(ws[e >> 1] >> ((e & 1) * 16));
      }
    } else {  // bf16 in, E4M3 out
      const uint4 w = in.w[0];
      const float inv = (kv ? c.v_inv_scale : c.k_inv_scale)[h];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      uint32_t code[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // one IEEE float32 multiply per element, then one rounding into E4M3
        code[2 * e] = f32_to_e4m3(__fmul_rn(bf16_lo(ws[e]), inv));
        code[2 * e + 1] = f32_to_e4m3(__fmul_rn(bf16_hi(ws[e]), inv));
      }
      uint8_t* pool = static_cast<uint8_t*>(c.pool);
      if (!kv) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo |= code[e] << (8 * e);
          hi |= code[4 + e] << (8 * e);
        }
        *reinterpret_cast<uint2*>(pool + dst) = make_uint2(lo, hi);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) pool[dst + e * step] = uint8_t(code[e]);
      }
    }
  }
}

// ---- MXFP4 ----------------------------------------------------------------------------
// Encoding of one 32-element block (OCP Microscaling conversion, as the cache
// description states it): one shared power-of-two scale, then every element rounded
// onto the E2M1 grid 0, .5, 1, 1.5, 2, 3, 4, 6 (mx_encode32).
struct MxCodes {
  uint32_t w[4];  // nibble e of w[c] = code of element 8c + e
  uint32_t scale;
};

// Two values (low nibble: a) into byte `byte` of `w` as E2M1 codes of value / scale:
// the hardware conversion rounds to nearest on the E2M1 grid with ties to the even
// code, clamps magnitudes above 6 to 6, keeps the sign (of zero too) and handles
// subnormal inputs exactly; it reads only the exponent field of `scale`.
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t w, float a, float b, float scale, int byte) {
  switch (byte) {  // the byte select is an immediate
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, scale, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, scale, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, scale, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, scale, 3);
  }
}

// 32 consecutive bf16 values (load32: 64-byte aligned).  The scale byte is max(E - 2,
// 0), E the bf16 exponent field of the largest magnitude (floor(log2) of a normal value
// is E - 127; a zero or subnormal maximum takes the clamp, byte 0 = 2^-127); each
// element is then x / 2^(byte - 127) rounded onto the E2M1 grid (e2m1_pair).  The
// scale passed to the conversion is the float whose exponent field is the byte (for
// byte 0 that is +0.0, whose exponent field 0 the conversion reads as 2^-127).
struct Bf16x32 {
  uint4 v[4];
};

__device__ __forceinline__ Bf16x32 load32(const uint16_t* __restrict__ src) {
  Bf16x32 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = reinterpret_cast<const uint4*>(src)[i];
  return r;
}

__device__ __forceinline__ MxCodes mx_encode32(const Bf16x32& x) {
  uint32_t h[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = x.v[i];
    h[4 * i] = v.x;
    h[4 * i + 1] = v.y;
    h[4 * i + 2] = v.z;
    h[4 * i + 3] = v.w;
  }
  uint32_t amax = 0;  // largest magnitude as bf16 bits (ordered like the values)
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, max(h[i] & 0x7fffu, (h[i] >> 16) & 0x7fffu));
  const uint32_t E = amax >> 7;
  MxCodes r;
  r.scale = E >= 2 ? E - 2 : 0;
  const float scale = __uint_as_float(r.scale << 23);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t w = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t bits = h[4 * c + p];  // elements 8c + 2p (low half) and 8c + 2p + 1
      w = e2m1_pair(w, __uint_as_float(bits << 16), __uint_as_float(bits & 0xffff0000u), scale, p);
    }
    r.w[c] = w;
  }
  return r;
}

// MXFP4 append: one 64-thread workgroup per packed row; a thread encodes one 32-dim
// block of one (K|V, kv head) row.  K blocks go to the token's own row (four words and
// a scale byte).  Two consecutive slots 2i, 2i+1 share their V code bytes (one nibble
// each), so the V bytes of a pair are written by one thread only: the row of the
// pair's first token that is new in this call.  It encodes every new token of the pair
// and keeps the nibble of a token that is not (already cached, or not yet written).
__global__ __launch_bounds__(64) void kv_append_mx_kernel(CacheArgs c, SeqArgs sq,
                                                          const uint16_t* __restrict__ k_new,
                                                          const uint16_t* __restrict__ v_new,
                                                          const int32_t* __restrict__ cu) {
  if (halted(c)) return;
  const int row = blockIdx.x;
  const int D = c.head_dim, H = c.num_kv_heads, P = c.page_size, J = D / 32;
  // The row's own K or V block of the first item, loaded before the slot lookup (it
  // depends on the row alone) so that its latency overlaps the lookup's loads.
  const int i0 = threadIdx.x;
  Bf16x32 own{};
  if (i0 < 2 * H * J) {
    const int kv = i0 >= H * J;
    const int hj = i0 - kv * H * J;
    own = load32((kv ? v_new : k_new) + int64_t(row) * H * D + hj * 32);
  }
  const int s = owner_of(cu, sq.num_seqs, row);
  const int first = cu[s], n = cu[s + 1] - first;
  const int L = sq.context_lens[s], pos0 = L - n;
  const int pos = pos0 + (row - first);
  const int32_t* bt = sq.block_tables + int64_t(s) * sq.max_pages_per_seq;
  const int64_t tb = tile_bytes(DT_MXFP4, P, D);
  uint8_t* pool = static_cast<uint8_t*>(c.pool);
  const int32_t page = bt[pos >> c.log2_page];
  const int slot = pos & (P - 1);
  const bool v_owner = !(pos & 1) || pos - 1 < pos0;
  for (int i = i0; i < 2 * H * J; i += blockDim.x) {
    const int kv = i >= H * J;
    const int hj = i - kv * H * J;
    const int h = hj / J, j = hj - (hj / J) * J;
    uint8_t* tile = pool + ((int64_t(page) * 2 + kv) * H + h) * tb;
    if (!kv) {
      const MxCodes e = mx_encode32(i == i0 ? own : load32(k_new + (int64_t(row) * H + h) * D + 32 * j));
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<uint32_t*>(tile + mx_k_word(slot, 32 * j + 8 * q, D)) = e.w[q];
      tile[mx_k_scale(P, slot, j, D)] = uint8_t(e.scale);
    } else if (v_owner) {
      const int pb = pos & ~1, sl = slot & ~1;  // the pair's first position and slot
      MxCodes e[2];
      bool fresh[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = pb + u;
        fresh[u] = p >= pos0 && p < L;
        if (fresh[u]) {
          e[u] = mx_encode32(p == pos && i == i0 ? own
                                                 : load32(v_new + (int64_t(first + p - pos0) * H + h) * D + 32 * j));
          tile[mx_v_scale(P, sl + u, j, D)] = uint8_t(e[u].scale);
        } else {
          e[u] = MxCodes{{0u, 0u, 0u, 0u}, 0u};
        }
      }
      const uint32_t keep = (fresh[0] ? 0u : 0x0fu) | (fresh[1] ? 0u : 0xf0u);
      // The 32 bytes are distinct (one per dim): every old byte is read before any is
      // written, so the reads are in flight together rather than one per round trip.
      uint32_t old[32] = {};
      if (keep) {
#pragma unroll
        for (int d = 0; d < 32; ++d) old[d] = tile[mx_v_byte(sl, 32 * j + d, D)];
      }
#pragma unroll
      for (int d = 0; d < 32; ++d) {
        const uint32_t lo = (e[0].w[d >> 3] >> (4 * (d & 7))) & 15u;  // low nibble: slot sl, high: sl + 1
        const uint32_t hi = (e[1].w[d >> 3] >> (4 * (d & 7))) & 15u;
        tile[mx_v_byte(sl, 32 * j + d, D)] = uint8_t((old[d] & keep) | ((lo | (hi << 4)) & ~keep));
      }
    }
  }
}

// MXFP4 gather: one workgroup per (4-token block, sequence); a thread writes one 32-dim
// block of one logical (token, K|V, head) row -- its 16 code bytes in dim order and its
// scale byte -- reading the tile through the same offset functions as the append.
__global__ __launch_bounds__(256) void debug_gather_mx_kernel(CacheArgs c, SeqArgs sq,
                                                              uint8_t* __restrict__ k_out,
                                                              uint8_t* __restrict__ v_out) {
  if (halted(c)) return;
  const int s = blockIdx.y;
  const int L = sq.context_lens[s];
  const int D = c.head_dim, H = c.num_kv_heads, P = c.page_size, J = D / 32;
  const int row_bytes = D / 2 + J;
  const int64_t tb = tile_bytes(DT_MXFP4, P, D);
  const int32_t* bt = sq.block_tables + int64_t(s) * sq.max_pages_per_seq;
  const uint8_t* pool = static_cast<const uint8_t*>(c.pool);
  const int t0 = blockIdx.x * 4;
  for (int i = threadIdx.x; i < 4 * 2 * H * J; i += blockDim.x) {
    const int tt = i / (2 * H * J);
    const int t = t0 + tt;
    if (t >= L) continue;
    const int rem = i - tt * 2 * H * J;
    const int kv = rem >= H * J;
    const int hj = rem - kv * H * J;
    const int h = hj / J, j = hj - (hj / J) * J;
    const int slot = t & (P - 1);
    const uint8_t* tile = pool + ((int64_t(bt[t >> c.log2_page]) * 2 + kv) * H + h) * tb;
    uint8_t* out = (kv ? v_out : k_out) + ((int64_t(s) * sq.max_context_len + t) * H + h) * row_bytes;
    for (int b = 0; b < 16; ++b) {
      uint32_t two = 0;
      for (int u = 0; u < 2; ++u) {
        const int d = 32 * j + 2 * b + u;
        uint32_t nib;
        if (!kv) {
          nib = (*reinterpret_cast<const uint32_t*>(tile + mx_k_word(slot, d, D)) >> (4 * (d & 7))) & 15u;
        } else {
          nib = (uint32_t(tile[mx_v_byte(slot, d, D)]) >> (4 * (vpos(slot & 31) & 1))) & 15u;
        }
        two |= nib << (4 * u);
      }
      out[16 * j + b] = uint8_t(two);
    }
    out[D / 2 + j] = tile[kv ? mx_v_scale(P, slot, j, D) : mx_k_scale(P, slot, j, D)];
  }
}

// Gather: one workgroup per (4-token block, sequence); each thread writes 16 bytes of
// one logical (token, K|V, head) row, read from the row (K) or column (V) of the tile.
__global__ __launch_bounds__(256) void debug_gather_kernel(CacheArgs c, SeqArgs sq,
                                                           uint8_t* __restrict__ k_out,
                                                           uint8_t* __restrict__ v_out) {
  if (halted(c)) return;
  const int s = blockIdx.y;
  const int L = sq.context_lens[s];
  const int eb = c.dtype == DT_F32 ? 4 : (c.dtype == DT_BF16 ? 2 : 1);
  const int row_bytes = c.head_dim * eb;
  const int vec_per_head = row_bytes / 16;
  const int vec_per_tok = c.num_kv_heads * vec_per_head;
  const int per16 = 16 / eb;  // elements per 16 bytes
  const int32_t* bt = sq.block_tables + int64_t(s) * sq.max_pages_per_seq;
  const uint8_t* pool = static_cast<const uint8_t*>(c.pool);
  const int t0 = blockIdx.x * 4;
  for (int i = threadIdx.x; i < 4 * 2 * vec_per_tok; i += blockDim.x) {
    const int tt = i / (2 * vec_per_tok);
    const int t = t0 + tt;
    if (t >= L) continue;
    const int rem = i - tt * 2 * vec_per_tok;
    const int kv = rem >= vec_per_tok;
    const int j = rem - kv * vec_per_tok;
    const int h = j / vec_per_head;
    const int d0 = (j - h * vec_per_head) * per16;
    const int64_t dst = ((int64_t(s) * sq.max_context_len + t) * c.num_kv_heads + h) * row_bytes + d0 * eb;
    uint8_t* out = (kv ? v_out : k_out) + dst;
    const int64_t src = elem_offset(bt, t, c.log2_page, kv, h, c.num_kv_heads, c.head_dim, d0) * eb;
    if (!kv) {
      *reinterpret_cast<uint4*>(out) = *reinterpret_cast<const uint4*>(pool + src);
    } else {
      const int64_t stride = int64_t(eb) << v_sub_log2(c.log2_page);
      for (int e = 0; e < per16; ++e)
        for (int b = 0; b < eb; ++b) out[e * eb + b] = pool[src + e * stride + b];
    }
  }
}

// Copy whole pages: page dst[i] <- page src[i], for i < n.  A page ([2][Hkv][tile]) is
// one contiguous range of the pool, so the copy is a plain 16-byte-vector copy;
// blockIdx.y = pair i, blockIdx.x strides over the page's 16-byte words.
__global__ __launch_bounds__(256) void copy_pages_kernel(uint4* __restrict__ pool, const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst, int64_t words,
                                                          const int32_t* __restrict__ flag) {
  if (flag && *flag) return;
  const int i = blockIdx.y;
  const int64_t s = src[i], d = dst[i];
  if (s == d) return;
  const uint4* from = pool + s * words;
  uint4* to = pool + d * words;
  for (int64_t w = int64_t(blockIdx.x) * 256 + threadIdx.x; w < words; w += int64_t(gridDim.x) * 256) to[w] = from[w];
}

}  // namespace

hipError_t launch_copy_pages(const CacheArgs& c, const int32_t* src, const int32_t* dst, int n,
                             hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t words = int64_t(2) * c.num_kv_heads * tile_bytes(c.dtype, c.page_size, c.head_dim) / 16;
  const int64_t per = std::min<int64_t>(64, (words + 255) / 256);  // workgroups per page
  hipLaunchKernelGGL(copy_pages_kernel, dim3(unsigned(per), unsigned(n)), dim3(256), 0, stream,
                     static_cast<uint4*>(c.pool), src, dst, words, c.debug_flag);
  return hipGetLastError();
}

hipError_t launch_kv_append(const CacheArgs& c, const SeqArgs& s, const void* k_new,
                            const void* v_new, int in_dtype, const int32_t* cu_new_lens,
                            int total_new, hipStream_t stream) {
  if (total_new == 0) return hipSuccess;
  const dim3 grid(total_new), block(256);
  if (c.dtype == DT_F32 && in_dtype == DT_F32)
    hipLaunchKernelGGL((kv_append_kernel<DT_F32, DT_F32>), grid, block, 0, stream, c, s, k_new, v_new, cu_new_lens);
  else if (c.dtype == DT_BF16 && in_dtype == DT_BF16)
    hipLaunchKernelGGL((kv_append_kernel<DT_BF16, DT_BF16>), grid, block, 0, stream, c, s, k_new, v_new, cu_new_lens);
  else if (c.dtype == DT_FP8 && in_dtype == DT_BF16)
    hipLaunchKernelGGL((kv_append_kernel<DT_BF16, DT_FP8>), grid, block, 0, stream, c, s, k_new, v_new, cu_new_lens);
  else if (c.dtype == DT_MXFP4 && in_dtype == DT_BF16)
    hipLaunchKernelGGL(kv_append_mx_kernel, grid, dim3(64), 0, stream, c, s, static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), cu_new_lens);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_debug_gather(const CacheArgs& c, const SeqArgs& s, void* k_out, void* v_out,
                               hipStream_t stream) {
  if (s.num_seqs == 0) return hipSuccess;
  const dim3 grid((s.max_context_len + 3) / 4, s.num_seqs), block(256);
  if (c.dtype == DT_MXFP4)
    hipLaunchKernelGGL(debug_gather_mx_kernel, grid, block, 0, stream, c, s, static_cast<uint8_t*>(k_out),
                       static_cast<uint8_t*>(v_out));
  else
    hipLaunchKernelGGL(debug_gather_kernel, grid, block, 0, stream, c, s,
                       static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out));
  return hipGetLastError();
}

}  // namespace pkv
