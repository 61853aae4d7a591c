// Causal prefill-chunk attention over the page pool on the matrix cores.
//
// What it computes: query i of sequence s's chunk of C queries sits at position
// L_s - C + i and attends to keys 0 .. that position, the chunk's own K/V included
// (appended before the call): a long prompt is cut into chunks, each appends its K/V
// and attends to everything before it ("NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践",
// §8), and context requests come first in the packed batch (§6).
//
// Here the contraction is dense (C queries x G heads share every K/V block), so both
// products run on the MFMA units.  The 16 MFMA rows of a tile are 16/G consecutive
// queries x the G heads of one kv head; a wave carries kPrefillTiles tiles, so every
// K/V block it loads (one 32-token block, straight into operand registers, the same
// loads as decode) feeds kPrefillTiles x 16 rows.  Causality is a per-row key limit,
// applied only on the blocks that reach a row's position.
//
// Work item (one wave): (sequence, kv head, key split, query tile).  When the chunk
// alone does not give enough waves to fill the device, each tile's key range is cut
// into equal block ranges (splits), whose normalised partials and log-sum-exps are
// merged exactly by a second kernel.  Workgroups go to the XCDs round robin; the
// grid is ordered so that all query tiles of one (sequence, kv head, split) land on
// the same XCD and read the same K/V blocks through its L2.
#include "mfma_common.h"

namespace pkv {
namespace {

constexpr int kPrefillTiles = 4;  // 16-row tiles per wave
constexpr int kXcds = 8;

// Query tile geometry for G query heads per kv head.
template <int G>
struct PfGeom {
  static constexpr int QPT = 16 / G;                 // queries per 16-row tile
  static constexpr int QW = kPrefillTiles * QPT;     // queries per wave
};

template <int KV, int D, int G, bool SMALLP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_kernel(AttnArgs a) {
  constexpr int NT = kPrefillTiles, QPT = PfGeom<G>::QPT, QW = PfGeom<G>::QW;
  const int lane = threadIdx.x, n = lane & 15, c = lane >> 4;
  const int Hkv = a.cache.num_kv_heads, Hq = a.num_q_heads, nsplit = a.max_splits;
  const int QT = a.pf_qtiles;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int grp = xcd + kXcds * (slot / QT), qt = slot % QT;
  if (grp >= a.seqs.num_seqs * Hkv * nsplit) return;
  const int split = grp % nsplit, sg = grp / nsplit;
  const int g = sg % Hkv, s = sg / Hkv;
  const int cq0 = a.cu_q_lens[s], C = a.cu_q_lens[s + 1] - cq0;
  const int q0 = qt * QW;
  if (q0 >= C) return;
  const int L = a.seqs.context_lens[s];
  const int pos0 = L - C;                          // position of query 0 of the chunk
  const int kend = pos0 + min(C, q0 + QW);         // keys [0, kend) reach this tile
  const int nb = (kend + BT - 1) >> LOG2_BT;
  const int b0 = int(int64_t(nb) * split / nsplit), b1 = int(int64_t(nb) * (split + 1) / nsplit);

  float qk_scale, vscale;
  scales<KV>(a, g, qk_scale, vscale);
  // Q^T operands and key limits: lane (n, c) of tile r is row n = query q0 + r*QPT +
  // n/G, head g*G + n%G; it sees keys t < lim[r] (0 for rows past the chunk).
  bf16x8 qf[NT][D / 32];
  int lim[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const int qi = q0 + r * QPT + n / G;
    lim[r] = qi < C ? pos0 + qi + 1 : 0;
    if (qi < C) {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (int64_t(cq0 + qi) * Hq + g * G + n % G) * D + 8 * c;
#pragma unroll
      for (int j = 0; j < D / 32; ++j) {
        Frag8 f;
        f.q = *reinterpret_cast<const uint4*>(qp + 32 * j);
        qf[r][j] = f.v;
      }
    } else {
#pragma unroll
      for (int j = 0; j < D / 32; ++j) qf[r][j] = zero8();
    }
  }
  const int lim_min = pos0 + q0 + 1;  // smallest limit of the tile's live rows
  State<D> st[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) state_init(st[r]);

  if (b0 < b1) {
    constexpr int esz = KV == DT_BF16 ? 2 : 1;
    const int64_t tile_b = int64_t(a.cache.page_size) * D * esz;
    const int32_t* bt = a.seqs.block_tables + int64_t(s) * a.seqs.max_pages_per_seq;
    run_blocks<KV, D, SMALLP>(
        static_cast<const char*>(a.cache.pool), bt, b0, b1, L, a.cache.log2_page, Hkv * tile_b,
        g * tile_b, lane, [&](Block<D>& blk, int t) {
          if (t + BT > L) mask_v_tail<D>(blk, L - t, lane);
#pragma unroll
          for (int r = 0; r < NT; ++r) {
            float sc[8];
            block_scores<D>(blk, qf[r], qk_scale, sc);
            if (t + BT > lim_min) {  // wave-uniform: the block reaches some row's position
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (t + tok_of(c, e) >= lim[r]) sc[e] = -INFINITY;
            }
            softmax_pv<D>(st[r], blk, sc, lane);
          }
        });
  }

  // finish every tile: rows of the chunk only
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    float l = st[r].l;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float lse = l > 0.f ? (st[r].m + __log2f(l)) * kLn2 : -INFINITY;  // row n
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lr = __shfl(l, 4 * c + i, 64);
      inv[i] = lr > 0.f ? vscale / lr : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // O rows 4c+i of this lane
      const int R = 4 * c + i;
      const int qi = q0 + r * QPT + R / G, h = R % G;
      if (qi >= C) continue;
      const int64_t row = cq0 + qi;
      if (nsplit == 1) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + (row * Hq + g * G + h) * D + n;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[16 * dt] = uint16_t(f32_to_bf16(st[r].o[dt][i] * inv[i]));
      } else {
        const int64_t rec = (row * Hkv + g) * nsplit + split;
        float* o = a.ws_o + (rec * G + h) * D + n;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[16 * dt] = st[r].o[dt][i] * inv[i];
      }
    }
    const int qi = q0 + r * QPT + n / G;
    if (c == 0 && qi < C) {
      const int64_t row = cq0 + qi;
      if (nsplit == 1) {
        if (a.lse_out) a.lse_out[row * Hq + g * G + n % G] = lse;
      } else {
        a.ws_lse[((row * Hkv + g) * nsplit + split) * G + n % G] = lse;
      }
    }
  }
}

// Merge of the key splits of one (query row, kv head).
template <int D, int G>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(AttnArgs a) {
  const int Hkv = a.cache.num_kv_heads, nsplit = a.max_splits;
  const int row = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int64_t r0 = (int64_t(row) * Hkv + g) * nsplit;
  merge_partials<D, G>(a, row, g, nsplit, [r0](int i) { return r0 + i; });
}

template <int KV, int D, int G, bool SMALLP>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  const int groups = a.seqs.num_seqs * a.cache.num_kv_heads * a.max_splits;
  const int64_t grid = int64_t((groups + kXcds - 1) / kXcds) * kXcds * a.pf_qtiles;
  hipLaunchKernelGGL((prefill_kernel<KV, D, G, SMALLP>), dim3(unsigned(grid)), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL((prefill_merge_kernel<D, G>), dim3(unsigned(int64_t(a.total_q) * a.cache.num_kv_heads)),
                     dim3(kMergeThreads), 0, st, a);
  return hipGetLastError();
}

template <int KV, int D, int G>
hipError_t dispatch_p(const AttnArgs& a, hipStream_t st) {
  return a.cache.page_size >= BT ? launch_t<KV, D, G, false>(a, st) : launch_t<KV, D, G, true>(a, st);
}

template <int KV, int D>
hipError_t dispatch_g(const AttnArgs& a, hipStream_t st) {
  switch (a.num_q_heads / a.cache.num_kv_heads) {
    case 1: return dispatch_p<KV, D, 1>(a, st);
    case 2: return dispatch_p<KV, D, 2>(a, st);
    case 4: return dispatch_p<KV, D, 4>(a, st);
    case 8: return dispatch_p<KV, D, 8>(a, st);
    case 16: return dispatch_p<KV, D, 16>(a, st);
  }
  return hipErrorInvalidValue;
}

template <int KV>
hipError_t dispatch_d(const AttnArgs& a, hipStream_t st) {
  return a.cache.head_dim == 64 ? dispatch_g<KV, 64>(a, st) : dispatch_g<KV, 128>(a, st);
}

}  // namespace

int mfma_prefill_queries_per_wave(int group) { return kPrefillTiles * (16 / group); }

int mfma_prefill_waves(int kv_dtype, int head_dim) {
  const void* k = kv_dtype == DT_BF16
                      ? (head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<DT_BF16, 64, 4, false>)
                                        : reinterpret_cast<const void*>(&prefill_kernel<DT_BF16, 128, 4, false>))
                      : (head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<DT_FP8, 64, 4, false>)
                                        : reinterpret_cast<const void*>(&prefill_kernel<DT_FP8, 128, 4, false>));
  return resident_blocks(k, 64);
}

hipError_t launch_mfma_prefill(const AttnArgs& a, hipStream_t st) {
  if (a.seqs.num_seqs == 0 || a.total_q == 0) return hipSuccess;
  return a.cache.dtype == DT_BF16 ? dispatch_d<DT_BF16>(a, st) : dispatch_d<DT_FP8>(a, st);
}

}  // namespace pkv
