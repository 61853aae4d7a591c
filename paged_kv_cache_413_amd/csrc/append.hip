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
// element per dim.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace pkv {
namespace {

// Sequence that owns packed row `row`: the largest s with cu[s] <= row.
__device__ __forceinline__ int owner_of(const int32_t* __restrict__ cu, int num_seqs, int row) {
  int lo = 0, hi = num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

template <int IN, int KV>
__global__ __launch_bounds__(256) void kv_append_kernel(CacheArgs c, SeqArgs sq,
                                                        const void* __restrict__ k_new,
                                                        const void* __restrict__ v_new,
                                                        const int32_t* __restrict__ cu) {
  const int row = blockIdx.x;
  const int s = owner_of(cu, sq.num_seqs, row);
  const int n = cu[s + 1] - cu[s];
  const int pos = sq.context_lens[s] - n + (row - cu[s]);
  const int32_t* bt = sq.block_tables + int64_t(s) * sq.max_pages_per_seq;
  const int D = c.head_dim, H = c.num_kv_heads;
  const int vec_per_head = D / 8;
  const int vec_per_row = H * vec_per_head;
  const int log2P = c.log2_page;
  for (int i = threadIdx.x; i < 2 * vec_per_row; i += blockDim.x) {
    const int kv = i >= vec_per_row;
    const int j = i - kv * vec_per_row;
    const int h = j / vec_per_head;
    const int e0 = (j - h * vec_per_head) * 8;
    const int64_t src = (int64_t(row) * H + h) * D + e0;
    const void* in = kv ? v_new : k_new;
    // K rows are contiguous in the tile (one vector store); V is dim-major inside its
    // sub-block, so the eight elements go to eight consecutive dims, one sub-block
    // length apart.
    const int64_t dst = elem_offset(bt, pos, log2P, kv, h, H, D, e0);
    const int64_t step = kv ? (int64_t(1) << v_sub_log2(log2P)) : 1;
    if constexpr (KV == DT_F32) {
      const float4* s4 = reinterpret_cast<const float4*>(static_cast<const float*>(in) + src);
      float* pool = static_cast<float*>(c.pool);
      if (!kv) {
        float4* d4 = reinterpret_cast<float4*>(pool + dst);
        d4[0] = s4[0];
        d4[1] = s4[1];
      } else {
        const float4 a = s4[0], b = s4[1];
        const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) pool[dst + e * step] = x[e];
      }
    } else if constexpr (KV == DT_BF16) {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + src);
      uint16_t* pool = static_cast<uint16_t*>(c.pool);
      if (!kv) {
        *reinterpret_cast<uint4*>(pool + dst) = w;
      } else {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) pool[dst + e * step] = uint16_t(ws[e >> 1] >> ((e & 1) * 16));
      }
    } else {  // bf16 in, E4M3 out
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + src);
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

// Gather: one workgroup per (4-token block, sequence); each thread writes 16 bytes of
// one logical (token, K|V, head) row, read from the row (K) or column (V) of the tile.
__global__ __launch_bounds__(256) void debug_gather_kernel(CacheArgs c, SeqArgs sq,
                                                           uint8_t* __restrict__ k_out,
                                                           uint8_t* __restrict__ v_out) {
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
                                                          const int32_t* __restrict__ dst, int64_t words) {
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
  const int esz = c.dtype == DT_F32 ? 4 : c.dtype == DT_BF16 ? 2 : 1;
  const int64_t words = int64_t(2) * c.num_kv_heads * c.page_size * c.head_dim * esz / 16;
  const int64_t per = std::min<int64_t>(64, (words + 255) / 256);  // workgroups per page
  hipLaunchKernelGGL(copy_pages_kernel, dim3(unsigned(per), unsigned(n)), dim3(256), 0, stream,
                     static_cast<uint4*>(c.pool), src, dst, words);
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
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_debug_gather(const CacheArgs& c, const SeqArgs& s, void* k_out, void* v_out,
                               hipStream_t stream) {
  if (s.num_seqs == 0) return hipSuccess;
  const dim3 grid((s.max_context_len + 3) / 4, s.num_seqs), block(256);
  hipLaunchKernelGGL(debug_gather_kernel, grid, block, 0, stream, c, s,
                     static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out));
  return hipGetLastError();
}

}  // namespace pkv
