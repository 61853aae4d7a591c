// Attention over the page pool on the vector ALUs: the general kernel.
//
// It serves every supported combination (f32 / bf16 / FP8 caches, f32 or bf16
// queries, head_dim 64 or 128, GQA groups 1..8), both decode rows and causal
// prefill rows.
//
// What it computes (per query row and head):  z_t = scale * q . K_t over the keys
// the row may see, softmax over z, output = sum_t softmax_t V_t.  A decode step
// reads the whole history ("NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践",
// §2); a prefill-chunk row sees keys up to its own position (§8).
//
// Work item = (row, kv head g, partition).  A partition is a page-aligned range of
// `chunk` keys; every partition keeps a running max / running sum (online softmax)
// and writes a normalised partial output with its log-sum-exp, merged exactly by
// merge_kernel.  A row whose keys fit one partition writes its output directly.
//
// Inside a workgroup (4 waves): a token row of D elements is read by D/8 lanes, 8
// elements each (16-byte loads of the token-major K tile; the dim-major V tile is read
// element by element), so one wave covers 64/(D/8) consecutive tokens per step.  This
// kernel is the general fallback (f32 caches and queries, pages shorter than 8
// tokens, prefill rows); the matrix-core kernel serves the bandwidth-critical shapes.  The q.K partial dot products are summed across the D/8 lanes with
// cross-lane shuffles; each group of D/8 lanes runs its own online softmax over its
// tokens, and the groups are merged once at the end (shuffles, then LDS across waves).
#include "device_common.h"
#include "internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;

template <int KV>
__device__ __forceinline__ void load8(const void* __restrict__ base, int64_t off, float (&x)[8]) {
  if constexpr (KV == DT_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else if constexpr (KV == DT_BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + off);
    fp8x2_to_f32(w.x, false, x[0], x[1]);
    fp8x2_to_f32(w.x, true, x[2], x[3]);
    fp8x2_to_f32(w.y, false, x[4], x[5]);
    fp8x2_to_f32(w.y, true, x[6], x[7]);
  }
}

// Eight elements `stride` apart: eight consecutive dims of one token in the V tile
// (dim-major inside its sub-block).
template <int KV>
__device__ __forceinline__ void load8_strided(const void* __restrict__ base, int64_t off,
                                              int64_t stride, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (KV == DT_F32) {
      x[e] = static_cast<const float*>(base)[off + e * stride];
    } else if constexpr (KV == DT_BF16) {
      x[e] = __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[off + e * stride]) << 16);
    } else {
      float a, b;
      fp8x2_to_f32(uint32_t(static_cast<const uint8_t*>(base)[off + e * stride]), false, a, b);
      x[e] = a;
    }
  }
}

template <int QT>
__device__ __forceinline__ void load_q8(const void* __restrict__ q, int64_t off, float (&x)[8]) {
  load8<QT == DT_F32 ? DT_F32 : DT_BF16>(q, off, x);
}

template <int QT>
__device__ __forceinline__ void store_out(void* out, int64_t off, float v) {
  if constexpr (QT == DT_F32) static_cast<float*>(out)[off] = v;
  else static_cast<uint16_t*>(out)[off] = uint16_t(f32_to_bf16(v));
}

// Sequence owning packed prefill row r.
__device__ __forceinline__ int owner_of(const int32_t* __restrict__ cu, int num_seqs, int row) {
  int lo = 0, hi = num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

// Combine two online-softmax states (log2 domain); an empty state has m = -inf.
__device__ __forceinline__ void combine(float& m, float& l, float* acc, float mo, float lo,
                                        const float* acco) {
  const float M = fmaxf(m, mo);
  const float a = (m == -INFINITY) ? 0.f : exp2f(m - M);
  const float b = (mo == -INFINITY) ? 0.f : exp2f(mo - M);
  l = l * a + lo * b;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a + acco[e] * b;
  m = M;
}

template <int KV, int QT, int D, int G, bool PREFILL>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a) {
  if (halted(a.cache)) return;
  constexpr int LPR = D / 8;        // lanes per token row
  constexpr int RPW = 64 / LPR;     // token rows per wave per step
  const int Hkv = a.cache.num_kv_heads;
  const int Hq = a.num_q_heads;

  // blockIdx.x = (row * Hkv + g) * max_splits + split
  const int split = blockIdx.x % a.max_splits;
  const int rg = blockIdx.x / a.max_splits;
  const int g = rg % Hkv;
  const int row = rg / Hkv;

  int s, nkeys;
  if constexpr (PREFILL) {
    s = owner_of(a.cu_q_lens, a.seqs.num_seqs, row);
    const int C = a.cu_q_lens[s + 1] - a.cu_q_lens[s];
    nkeys = a.seqs.context_lens[s] - C + (row - a.cu_q_lens[s]) + 1;
  } else {
    s = row;
    nkeys = a.seqs.context_lens[s];
  }
  const int t0 = split * a.chunk;
  if (t0 >= nkeys) return;
  const int t1 = min(nkeys, t0 + a.chunk);
  const int nsplit = (nkeys + a.chunk - 1) / a.chunk;
  // keys before the window (a partition wholly before it keeps an empty state and
  // records lse = -inf and a zero output, which the merge skips)
  const int tlo = max(t0, window_lo(nkeys - 1, a.seqs.window));

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane / LPR, c = lane % LPR;
  const int32_t* bt = a.seqs.block_tables + int64_t(s) * a.seqs.max_pages_per_seq;
  const void* pool = a.cache.pool;
  const float qscale = a.sm_scale * kLog2e;
  float kscale = 1.f, vscale = 1.f;
  if constexpr (KV == DT_FP8) {
    kscale = a.cache.k_scale[g];
    vscale = a.cache.v_scale[g];
  }

  float q[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    load_q8<QT>(a.q, (int64_t(row) * Hq + g * G + h) * D + c * 8, q[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[h][e] *= qscale * kscale;
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  for (int tb = tlo + w * RPW; tb < t1; tb += kWaves * RPW) {
    const int t = tb + r;
    if (t < t1) {
      const int64_t koff = elem_offset(bt, t, a.cache.log2_page, 0, g, Hkv, D, c * 8);
      const int64_t voff = elem_offset(bt, t, a.cache.log2_page, 1, g, Hkv, D, c * 8);
      float k[8], v[8];
      load8<KV>(pool, koff, k);
      load8_strided<KV>(pool, voff, int64_t(1) << v_sub_log2(a.cache.log2_page), v);
      float sc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(q[h][e], k[e], d);
        sc[h] = d;
      }
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h] += __shfl_xor(sc[h], off, 64);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], sc[h]);
        const float corr = exp2f(m[h] - mn);
        const float p = exp2f(sc[h] - mn);
        l[h] = l[h] * corr + p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e] * corr);
        m[h] = mn;
      }
    }
  }

  // merge the RPW row groups of this wave (lanes with equal c)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off, 64);
      const float lo = __shfl_xor(l[h], off, 64);
      float ao[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ao[e] = __shfl_xor(acc[h][e], off, 64);
      combine(m[h], l[h], acc[h], mo, lo, ao);
    }
  }

  // merge the waves through LDS
  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[w][h][c * 8 + e] = acc[h][e];
      if (c == 0) {
        sm_m[w][h] = m[h];
        sm_l[w][h] = l[h];
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int h = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww][h]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = sm_m[ww][h];
      const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      lsum += f * sm_l[ww][h];
      osum += f * sm_acc[ww][h][d];
    }
    const float o = lsum > 0.f ? osum / lsum * vscale : 0.f;
    const float lse = (M + __log2f(lsum)) * kLn2;   // natural-log units
    const int hq = g * G + h;
    if (nsplit == 1) {
      store_out<QT>(a.out, (int64_t(row) * Hq + hq) * D + d, o);
      if (a.lse_out && d == 0) a.lse_out[int64_t(row) * Hq + hq] = lse;
    } else {
      const int64_t base = (int64_t(row) * Hq + hq) * a.max_splits + split;
      a.ws_o[base * D + d] = o;
      if (d == 0) a.ws_lse[base] = lse;
    }
  }
}

// Exact merge of the partitions of one (row, query head):
// LSE = log sum_j exp(lse_j), out = sum_j exp(lse_j - LSE) o_j.
template <int QT, bool PREFILL>
__global__ __launch_bounds__(128) void merge_kernel(AttnArgs a) {
  if (halted(a.cache)) return;
  const int hq = blockIdx.x % a.num_q_heads;
  const int row = blockIdx.x / a.num_q_heads;
  int nkeys;
  if constexpr (PREFILL) {
    const int s = owner_of(a.cu_q_lens, a.seqs.num_seqs, row);
    const int C = a.cu_q_lens[s + 1] - a.cu_q_lens[s];
    nkeys = a.seqs.context_lens[s] - C + (row - a.cu_q_lens[s]) + 1;
  } else {
    nkeys = a.seqs.context_lens[row];
  }
  const int n = (nkeys + a.chunk - 1) / a.chunk;
  if (n <= 1) return;  // written directly by the attention kernel
  const int D = a.cache.head_dim;
  const int64_t base = (int64_t(row) * a.num_q_heads + hq) * a.max_splits;
  float M = -INFINITY;
  for (int j = 0; j < n; ++j) M = fmaxf(M, a.ws_lse[base + j]);
  float wsum = 0.f;
  for (int j = 0; j < n; ++j) wsum += __expf(a.ws_lse[base + j] - M);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float o = 0.f;
    for (int j = 0; j < n; ++j)
      if (a.ws_lse[base + j] != -INFINITY) o += __expf(a.ws_lse[base + j] - M) * a.ws_o[(base + j) * D + d];
    store_out<QT>(a.out, (int64_t(row) * a.num_q_heads + hq) * D + d, o / wsum);
  }
  if (a.lse_out && threadIdx.x == 0) a.lse_out[int64_t(row) * a.num_q_heads + hq] = M + __logf(wsum);
}

template <int KV, int QT, int D, int G, bool PREFILL>
hipError_t launch_t(const AttnArgs& a, int rows, hipStream_t st) {
  const int64_t nblk = int64_t(rows) * a.cache.num_kv_heads * a.max_splits;
  hipLaunchKernelGGL((attn_valu_kernel<KV, QT, D, G, PREFILL>), dim3(unsigned(nblk)), dim3(256), 0,
                     st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL((merge_kernel<QT, PREFILL>), dim3(unsigned(int64_t(rows) * a.num_q_heads)),
                     dim3(128), 0, st, a);
  return hipGetLastError();
}

template <int KV, int QT, int D, bool PREFILL>
hipError_t dispatch_g(const AttnArgs& a, int rows, hipStream_t st) {
  switch (a.num_q_heads / a.cache.num_kv_heads) {
    case 1: return launch_t<KV, QT, D, 1, PREFILL>(a, rows, st);
    case 2: return launch_t<KV, QT, D, 2, PREFILL>(a, rows, st);
    case 4: return launch_t<KV, QT, D, 4, PREFILL>(a, rows, st);
    case 8: return launch_t<KV, QT, D, 8, PREFILL>(a, rows, st);
  }
  return hipErrorInvalidValue;
}

template <int KV, int QT, bool PREFILL>
hipError_t dispatch_d(const AttnArgs& a, int rows, hipStream_t st) {
  return a.cache.head_dim == 64 ? dispatch_g<KV, QT, 64, PREFILL>(a, rows, st)
                                : dispatch_g<KV, QT, 128, PREFILL>(a, rows, st);
}

template <bool PREFILL>
hipError_t dispatch(const AttnArgs& a, int rows, hipStream_t st) {
  const int kv = a.cache.dtype, qt = a.q_dtype;
  if (qt == DT_F32) {
    if (kv == DT_F32) return dispatch_d<DT_F32, DT_F32, PREFILL>(a, rows, st);
    if (kv == DT_BF16) return dispatch_d<DT_BF16, DT_F32, PREFILL>(a, rows, st);
    if (kv == DT_FP8) return dispatch_d<DT_FP8, DT_F32, PREFILL>(a, rows, st);
  } else {
    if (kv == DT_F32) return dispatch_d<DT_F32, DT_BF16, PREFILL>(a, rows, st);
    if (kv == DT_BF16) return dispatch_d<DT_BF16, DT_BF16, PREFILL>(a, rows, st);
    if (kv == DT_FP8) return dispatch_d<DT_FP8, DT_BF16, PREFILL>(a, rows, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool valu_supported(int kv_dtype, int q_dtype, int head_dim, int group) {
  return (kv_dtype == DT_F32 || kv_dtype == DT_BF16 || kv_dtype == DT_FP8) &&
         (q_dtype == DT_F32 || q_dtype == DT_BF16) && (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_valu_decode(const AttnArgs& a, hipStream_t st) {
  if (a.seqs.num_seqs == 0) return hipSuccess;
  return dispatch<false>(a, a.seqs.num_seqs, st);
}

hipError_t launch_valu_prefill(const AttnArgs& a, hipStream_t st) {
  if (a.total_q == 0) return hipSuccess;
  return dispatch<true>(a, a.total_q, st);
}

}  // namespace pkv
