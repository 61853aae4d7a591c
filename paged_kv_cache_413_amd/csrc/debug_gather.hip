// paged_kv_debug_gather_operands: the matrix-core attention kernels' own page loaders,
// run over every cached token, with the operands they produce written back in logical
// order -- so that the hot path's page-gather indexing (logical block -> physical page
// through the block table, "NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践", §9)
// can be compared bit for bit with a plain gather.
//
// Path 0 runs the decode kernels' block pipeline (run_blocks: the page window held in a
// register, per-tile buffer descriptors, blocks in flight) and writes each block as its
// registers hold it; path 2 the same pipeline with the dense FP8 decode kernel's raw
// blocks (widened when folded).  Path 1 runs the prefill kernel's staging (Stager: a workgroup
// fetches a block, decodes it to bf16 into LDS) and reads the operands back from the
// stage with the prefill kernel's lane map.  Values: bf16 caches as stored, FP8 codes
// widened exactly, MXFP4 elements times their block scale.
#include "stage.h"

namespace pkv {
namespace {

// Lane (m, c) of a block's K operands: tokens m (ka) and 16 + m (kb), dims 32j + 8c..+7
// of chunk j; of its V operands: dims 16dt + m, tokens tok_of(c, e).  Tokens at or past
// L are not written.
template <int D>
__device__ __forceinline__ void write_k(uint16_t* out, int64_t row0, int Hkv, int t, int L, int j, int half,
                                        bf16x8 v, int lane) {
  const int m = lane & 15, c = lane >> 4, tok = t + 16 * half + m;
  if (tok >= L) return;
  Frag8 f;
  f.v = v;
  *reinterpret_cast<uint4*>(out + ((row0 + tok) * Hkv) * D + 32 * j + 8 * c) = f.q;
}

__device__ __forceinline__ void write_v8(uint16_t* out, int64_t row0, int Hkv, int D, int t, int L, int dim,
                                         const uint32_t (&w)[4], int lane) {
  const int c = lane >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int tok = t + tok_of(c, e);
    if (tok < L) out[((row0 + tok) * Hkv) * D + dim] = uint16_t(w[e >> 1] >> (16 * (e & 1)));
  }
}

template <int KV, int D, bool SMALLP, bool RAW = false>
__global__ __launch_bounds__(64) void operands_decode_kernel(CacheArgs c, SeqArgs sq, uint16_t* __restrict__ k_out,
                                                             uint16_t* __restrict__ v_out) {
  if (halted(c)) return;
  const int lane = threadIdx.x;
  const int Hkv = c.num_kv_heads, g = blockIdx.x % Hkv, s = blockIdx.x / Hkv;
  const int L = uniform32(sq.context_lens[s]);
  const int64_t tile_b = tile_bytes(KV, c.page_size, D);
  const int32_t* bt = sq.block_tables + int64_t(s) * sq.max_pages_per_seq;
  const int64_t row0 = int64_t(s) * sq.max_context_len;  // row (s, t) of the outputs, kv head added below
  uint16_t* ko = k_out + int64_t(g) * D;
  uint16_t* vo = v_out + int64_t(g) * D;
  run_blocks<KV, D, SMALLP, RAW>(static_cast<const char*>(c.pool), bt, 0, (L + BT - 1) >> LOG2_BT, L, c.log2_page,
                            Hkv * tile_b, g * tile_b, lane, [&](auto& blk, int t) {
    const auto& r = ready<D>(blk);
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      write_k<D>(ko, row0, Hkv, t, L, j, 0, r.ka[j], lane);
      write_k<D>(ko, row0, Hkv, t, L, j, 1, r.kb[j], lane);
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      Frag8 f;
      f.v = r.v[dt];
      uint32_t w[4] = {f.w[0], f.w[1], f.w[2], f.w[3]};
      if constexpr (KV == DT_MXFP4) {
        // the codes' own scales, as the P.V product applies them to the weights: element
        // e of this lane is position 8c + e, 32-dim block dt / 2
        constexpr int J = D / 32;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int byte = e * J + dt / 2;
          const int ex = int((r.vs[byte >> 2] >> (8 * (byte & 3))) & 255u) - 127;
          const float x = __builtin_ldexpf(__uint_as_float((w[e >> 1] >> (16 * (e & 1))) << 16), ex);
          const uint32_t b = f32_to_bf16(x);
          w[e >> 1] = (w[e >> 1] & (0xffffu << (16 * (1 - (e & 1))))) | (b << (16 * (e & 1)));
        }
      }
      write_v8(vo, row0, Hkv, D, t, L, 16 * dt + (lane & 15), w, lane);
    }
  });
}

template <int KV, int D>
__global__ __launch_bounds__(kPfThreads) void operands_prefill_kernel(CacheArgs c, SeqArgs sq,
                                                                     uint16_t* __restrict__ k_out,
                                                                     uint16_t* __restrict__ v_out) {
  if (halted(c)) return;
  using SL = Stager<KV, D, kPfThreads>;
  __shared__ __attribute__((aligned(1024))) char smem[SL::BYTES];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int Hkv = c.num_kv_heads, g = blockIdx.x % Hkv, s = blockIdx.x / Hkv;
  const int L = uniform32(sq.context_lens[s]);
  const int64_t tile_b = tile_bytes(KV, c.page_size, D);
  const BlockSrc src{static_cast<const char*>(c.pool), sq.block_tables + int64_t(s) * sq.max_pages_per_seq,
                     c.log2_page, Hkv * tile_b, g * tile_b};
  const int64_t row0 = int64_t(s) * sq.max_context_len;
  uint16_t* ko = k_out + int64_t(g) * D;
  uint16_t* vo = v_out + int64_t(g) * D;
  const uint32_t lk = stage_lane_offset(lane);
  for (int blk = 0; blk < (L + BT - 1) >> LOG2_BT; ++blk) {
    const int t = blk << LOG2_BT;
    typename SL::Regs r;
    SL::fetch(r, src, blk, tid);
    SL::stash(r, smem, L - t, tid);
    __syncthreads();
    for (int j = w; j < D / 32; j += SL::NW) {
      write_k<D>(ko, row0, Hkv, t, L, j, 0, SL::k_operand(smem, j, 0, lk), lane);
      write_k<D>(ko, row0, Hkv, t, L, j, 1, SL::k_operand(smem, j, 1, lk), lane);
    }
    for (int dt = w; dt < D / 16; dt += SL::NW) {
      Frag8 f;
      f.v = SL::v_operand(smem, dt, lk);
      const uint32_t wd[4] = {f.w[0], f.w[1], f.w[2], f.w[3]};
      write_v8(vo, row0, Hkv, D, t, L, 16 * dt + (lane & 15), wd, lane);
    }
    __syncthreads();  // the stage is rewritten by the next block
  }
}

template <int KV, int D>
hipError_t launch_d(const CacheArgs& c, const SeqArgs& s, int path, uint16_t* k, uint16_t* v, hipStream_t st) {
  const dim3 grid(unsigned(int64_t(s.num_seqs) * c.num_kv_heads));
  if (path == 1) {
    if constexpr (KV != DT_F32) hipLaunchKernelGGL((operands_prefill_kernel<KV, D>), grid, dim3(kPfThreads), 0, st, c, s, k, v);
  } else if (path == 2) {
    if constexpr (KV == DT_FP8) hipLaunchKernelGGL((operands_decode_kernel<KV, D, false, true>), grid, dim3(64), 0, st, c, s, k, v);
  } else if (c.page_size >= BT) {
    hipLaunchKernelGGL((operands_decode_kernel<KV, D, false>), grid, dim3(64), 0, st, c, s, k, v);
  } else {
    if constexpr (KV != DT_MXFP4) hipLaunchKernelGGL((operands_decode_kernel<KV, D, true>), grid, dim3(64), 0, st, c, s, k, v);
  }
  return hipGetLastError();
}

template <int KV>
hipError_t launch_k(const CacheArgs& c, const SeqArgs& s, int path, uint16_t* k, uint16_t* v, hipStream_t st) {
  return c.head_dim == 64 ? launch_d<KV, 64>(c, s, path, k, v, st) : launch_d<KV, 128>(c, s, path, k, v, st);
}

}  // namespace

bool operands_supported(int kv_dtype, int page_size, int head_dim, int path) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (path == 2) return kv_dtype == DT_FP8 && page_size >= BT;
  if (kv_dtype == DT_MXFP4 || path == 1) return page_size >= BT && kv_dtype != DT_F32;
  return (kv_dtype == DT_BF16 || kv_dtype == DT_FP8) && page_size >= 8;
}

hipError_t launch_debug_operands(const CacheArgs& c, const SeqArgs& s, int path, void* k_out, void* v_out,
                                 hipStream_t st) {
  if (s.num_seqs == 0) return hipSuccess;
  uint16_t* k = static_cast<uint16_t*>(k_out);
  uint16_t* v = static_cast<uint16_t*>(v_out);
  switch (c.dtype) {
    case DT_BF16: return launch_k<DT_BF16>(c, s, path, k, v, st);
    case DT_FP8: return launch_k<DT_FP8>(c, s, path, k, v, st);
    case DT_MXFP4: return launch_k<DT_MXFP4>(c, s, path, k, v, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
