// Decode attention over the page pool on the matrix cores (bf16 MFMA, fp32 accumulate).
//
// What it computes (per sequence s and query head h): z_t = scale * q . K_t for every
// cached token t < L_s, softmax over z, output = sum_t softmax_t V_t.  A decode step
// appends the new token and then reads the whole history through the block table
// ("NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践", §2 and §9; "TensorRT-LLM",
// 关键机制, PagedAttention).
//
// Work unit: one wave (64 lanes) processes blocks of 32 consecutive tokens of one
// (sequence, kv head).  The G query heads that share the kv head form the 16 rows of
// the MFMA tiles (G <= 16; unused rows are zero), so per block:
//   scores^T [32 tok x 16 heads] = K [32 x D] . Q^T [D x 16]   -> 2 x D/32 MFMAs
//   O        [16 heads x D]     += P [16 x 32 tok] . V [32 x D] -> D/16 MFMAs
// Every operand comes straight from HBM in the register layout the MFMA wants:
//   K tile of a page is [D/32][P][32] (32-dim chunks, token-major inside a chunk):
//   lane (m, c) loads 8 dims of one token row, and the 16 token rows of one load are
//   one contiguous kilobyte;
//   V tile of a page is dim-major inside 32-slot sub-blocks [P/32][D][32]: lane (n, c)
//   loads 8 consecutive tokens of one dim, and the 16 dims of one load are one
//   contiguous kilobyte -- so no LDS transpose sits on the hot path.
// The two K sub-tiles are tokens 0..15 and 16..31 of the block, so the scores of
// head n land in lane (n, c) for tokens 4c..4c+3 and 16+4c..16+4c+3 -- exactly the P
// operand of the second product (k index 8c + e), so scores never leave their lanes;
// the V sub-block stores its slots in that same order.  The row max of the online
// softmax needs two cross-lane steps (lanes 16 and 32 apart); the running sum is
// kept per lane and reduced once per range.
//
// Schedule: "auto" spreads the flattened (sequence, kv head, block) space evenly over
// the resident waves (each wave a contiguous run of blocks, possibly spanning several
// sequences; each XCD takes a contiguous eighth of that order; FP8 calls with more
// segments than waves use the two-waves-per-SIMD "dense" variant with raw FP8 blocks);
// a range that covers a whole (sequence, kv head) writes the output
// directly, a cut one writes a normalised partial and its log-sum-exp, and a small
// merge kernel combines the pieces exactly (log-sum-exp weights).  "fixed" gives each
// page-aligned partition of a fixed size its own wave, as in a conventional split-KV
// decode, with the same merge.  (Merging inside the decode kernel, by the last wave
// to finish a piece, needs agent-scope release/acquire fences; on this chip those
// write back and invalidate a whole L2 per piece, which costs far more than the
// second launch.)
#include "mfma_common.h"

namespace pkv {
namespace {

// Keys a tile row sees: lo_row <= t < lim_row (its window start and causal limit; for
// decode 0 or the window start, and the sequence length), further cut to the range's
// t_end.  lim_min = min(t_end, smallest lim_row) and lo_max = largest lo_row are
// wave-uniform.
struct RowKeys {
  int t_end, lim_row, lim_min, lo_row, lo_max;
};

// Fold one block into the state of the tile's rows.  On the blocks that reach a row's
// limit or start before a row's window the excluded keys' scores are masked, and on the
// range's last, partial block the V entries past t_end are zeroed.  An MXFP4 or raw FP8
// block is decoded first (ready); a bf16 / widened FP8 one is used as loaded.
template <int D, typename Blk>
__device__ __forceinline__ void fold_block(State<D>& st, Blk& b, const bf16x8 (&qf)[D / 32],
                                           float qk_scale, int t, const RowKeys& k, int lane) {
  constexpr bool kRaw = std::is_same_v<Blk, F8Block<D>>;  // its tail is masked on the codes
  if constexpr (kRaw) {
    if (t + BT > k.t_end) mask_v_tail<D>(b, k.t_end - t, lane);
  }
  const auto& r = ready<D>(b);
  float sc[8];
  block_scores<D>(r, qf, sc);
  if (t + BT > k.lim_min || t < k.lo_max) {  // wave-uniform
    const int c = lane >> 4, lim = min(k.t_end, k.lim_row);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tk = t + tok_of(c, e);
      if (tk >= lim || tk < k.lo_row) sc[e] = -INFINITY;
    }
    if constexpr (!kRaw) {
      if (t + BT > k.t_end) mask_v_tail<D>(b, k.t_end - t, lane);
    }
  }
  softmax_pv<D>(st, r, sc, qk_scale, lane);
}

// Blocks [b0, b1) of one (sequence, kv head).
// win0: the block-table window of block b0's page, already loaded (or NULL).
template <int KV, int D, bool SMALLP, bool RAW = false>
__device__ __forceinline__ void run_range(State<D>& st, const bf16x8 (&qf)[D / 32], float qk_scale,
                                          const char* __restrict__ pool, const int32_t* __restrict__ bt,
                                          int b0, int b1, const RowKeys& k, int L, int log2P,
                                          int64_t kv_stride_b, int64_t head_off_b, int lane,
                                          const PageWindow* win0 = nullptr) {
  run_blocks<KV, D, SMALLP, RAW>(
      pool, bt, b0, b1, L, log2P, kv_stride_b, head_off_b, lane,
      [&](auto& b, int t) { fold_block<D>(st, b, qf, qk_scale, t, k, lane); }, win0);
}

// Finish a range: reduce the running sum over the four lane groups of each row and
// normalise.  Tile row R is query R / G of the sequence (packed row q0 + R / G) and
// head g*G + R % G; rows of queries >= nq are not written.  A range that covers its
// whole (sequence, kv head) writes the output (bf16) and log-sum-exp directly; a cut
// one writes partial record `rec`: ws_o[rec][ROWS][D] (normalised) and
// ws_lse[rec][ROWS], merged by the merge kernel.
template <int D, int G, int ROWS>
__device__ __forceinline__ void finish(const State<D>& st, const AttnArgs& a, int q0, int nq, int g,
                                       bool complete, int64_t rec, float qk_scale, float vscale,
                                       int lane) {
  const int nn = lane & 15, c = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const float lse = row_lse(st.m, l, qk_scale);  // natural log of row nn
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lr = __shfl(l, 4 * c + i, 64);
    inv[i] = lr > 0.f ? vscale / lr : 0.f;
  }
  const int Hq = a.num_q_heads;
  if (complete) {
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int R = 4 * c + i;
      if (R < ROWS && R / G < nq) {
        uint16_t* o = out + (int64_t(q0 + R / G) * Hq + g * G + R % G) * D + nn;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[16 * dt] = uint16_t(f32_to_bf16(st.o[dt][i] * inv[i]));
      }
    }
    if (a.lse_out && c == 0 && nn < ROWS && nn / G < nq)
      a.lse_out[int64_t(q0 + nn / G) * Hq + g * G + nn % G] = lse;
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int R = 4 * c + i;
    if (R < ROWS) {
      float* o = a.ws_o + (rec * ROWS + R) * D + nn;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[16 * dt] = st.o[dt][i] * inv[i];
    }
  }
  if (c == 0 && nn < ROWS) a.ws_lse[rec * ROWS + nn] = lse;
}

// Independent waves per workgroup of the decode kernels (no LDS, no barriers: a larger
// workgroup only packs them onto one CU, one per SIMD).  Placing 1024 one-wave
// workgroups takes the dispatcher about 4 us, but packing 2 or 4 measured no faster:
// the waves placed first already keep HBM busy.
#ifndef PKV_DECODE_WG_WAVES
#define PKV_DECODE_WG_WAVES 1
#endif
constexpr int kWgWaves = PKV_DECODE_WG_WAVES;

// Waves per SIMD the decode kernels are compiled for (bf16 / FP8: see
// PKV_DECODE_WAVES_PER_EU).  MXFP4 does several times the vector work per byte; two
// waves let one SIMD issue one wave's decoding while the other waits for its loads.
#ifndef PKV_MX_WAVES_PER_EU
#define PKV_MX_WAVES_PER_EU 2
#endif
template <int KV>
constexpr int kDecodeWavesPerEu = KV == DT_MXFP4 ? PKV_MX_WAVES_PER_EU : PKV_DECODE_WAVES_PER_EU;

// Dense FP8 decode (DENSE): raw FP8 blocks, widened when folded (half the registers of a
// widened block), and two waves per SIMD.  The host picks it for one-query FP8 calls with
// more (sequence, kv head) segments than one wave per SIMD gives waves: each wave then
// starts several segments, and every start is a chain of dependent loads (lengths, table
// window, first block) that a second wave on the SIMD covers.  Measured on the mixed
// batch's FP8 decode (2 048 segments): 185 -> 171 us; on 512 - 1 024 segments (Llama-shaped
// FP8 batches, the shared-prefix batch) it is 3 - 10 % slower, so those keep one wave.
template <int KV, bool DENSE>
constexpr int kAutoWavesPerEu = DENSE ? 2 : kDecodeWavesPerEu<KV>;

// ---- fixed partitions: one wave per (sequence, kv head, partition) ---------------------
template <int KV, int D, int G, bool SMALLP>
__global__ __launch_bounds__(64 * kWgWaves) __attribute__((amdgpu_waves_per_eu(kDecodeWavesPerEu<KV>, kDecodeWavesPerEu<KV>))) void decode_fixed_kernel(AttnArgs a) {
  if (halted(a.cache)) return;
  const int lane = threadIdx.x & 63;
  const int64_t wid = int64_t(blockIdx.x) * kWgWaves + uniform32(threadIdx.x >> 6);
  const int Hkv = a.cache.num_kv_heads;
  if (wid >= int64_t(a.seqs.num_seqs) * Hkv * a.max_splits) return;
  const int split = int(wid % a.max_splits);
  const int sg = int(wid / a.max_splits);
  const int g = sg % Hkv, s = sg / Hkv;
  const int L = uniform32(a.seqs.context_lens[s]);
  const int t0 = split * a.chunk;
  if (t0 >= L) return;
  const int t1 = min(L, t0 + a.chunk);
  const int nsplit = (L + a.chunk - 1) / a.chunk;
  // a partition wholly before the window keeps an empty state: it records lse = -inf
  // and zeros, which the merge skips
  const int lo = window_lo(L - 1, a.seqs.window), ts = max(t0, lo);
  float qk_scale, vscale;
  scales<KV>(a, g, qk_scale, vscale);
  bf16x8 qf[D / 32];
  load_q<D, G>(qf, a.q, s, 1, a.num_q_heads, g, lane);
  State<D> st;
  state_init(st);
  const int64_t tile_b = tile_bytes(KV, a.cache.page_size, D);
  const int32_t* bt = a.seqs.block_tables + int64_t(s) * a.seqs.max_pages_per_seq;
  if (ts < t1)
    run_range<KV, D, SMALLP>(st, qf, qk_scale, static_cast<const char*>(a.cache.pool), bt, ts >> LOG2_BT,
                             (t1 + BT - 1) >> LOG2_BT, RowKeys{t1, L, t1, lo, lo}, L, a.cache.log2_page,
                             Hkv * tile_b, g * tile_b, lane);
  finish<D, G, G>(st, a, s, 1, g, nsplit == 1, int64_t(sg) * a.max_splits + split, qk_scale, vscale, lane);
}

// ---- auto: contiguous equal shares of the flattened blocks (and segment start costs) --
// Flattened order: sequence-major, then kv head, then block.  Each (sequence, kv head)
// segment counts SC units more than its nb_s blocks: the cost of starting a segment (the
// wave's pipeline drains, the queries and first blocks are loaded, the result is
// written) in block times.  Segment (s, g) spans units [Hkv*cum_s + g*nu_s, +nu_s),
// nu_s = nb_s + SC, cum_s = sum_{s'<s} nu_s'; its first SC units hold no block, and its
// block k is unit Hkv*cum_s + g*nu_s + SC + k.  Waves take equal shares of units, so a
// wave whose share holds many short segments holds fewer blocks.  Equal shares of blocks
// alone left such waves behind (per-wave clocks, mixed batch: the last wave ended 47 us
// after the median one).  SC per kernel, measured (decode call, us, SC = 0 / 2 / 3 / 4):
// one wave per SIMD, bf16: Llama batch 98.1 / 97.7 / 99.1 / 99.5, mixed batch 301.2 /
// 288.7 / 284.9 / 285.6 -> 2; FP8: Llama-shaped batch - / 54.3 / 52.9 / 53.1 (the
// shared-prefix batch flat) -> 3; two waves per SIMD: dense FP8 mixed batch 169.0 /
// 157.6 / 155.0 / 153.5 (SC 6 / 8: 155.2 / 155.7) -> 4; MXFP4 Llama batch 40.0 / 39.4 /
// 38.8 / 38.6 (SC 5 / 6: 39.3 / 39.0), MXFP4 mixed batch SC 4 / 5 / 6 / 8: 97.4 / 95.6 /
// 93.7 / 95.2 -> 6.
template <int KV, bool DENSE>
constexpr int kSegCost = KV == DT_MXFP4 ? 6 : DENSE ? 4 : KV == DT_FP8 ? 3 : 2;

__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// Blocks of each (sequence, kv head) segment of sequence s: the 32-token blocks from
// the one holding the first key its earliest query sees to the one holding its last
// key (L tokens, nq queries at positions L - nq .. L - 1, window W); blo = the first.
__device__ __forceinline__ int seg_blocks(int L, int nq, int W, int& blo) {
  blo = window_lo(L - nq, W) >> LOG2_BT;
  return ((L + BT - 1) >> LOG2_BT) - blo;
}

// Units of a segment in the flattened order: its blocks and its start cost SC.
template <int SC>
__device__ __forceinline__ int seg_units(int L, int nq, int W) {
  int blo;
  return seg_blocks(L, nq, W, blo) + SC;
}

// Queries of sequence s in this call: packed rows cu[s] .. cu[s+1]-1, or the one row s.
__device__ __forceinline__ int queries_of(const int32_t* __restrict__ cu, int s) {
  return cu ? cu[s + 1] - cu[s] : 1;
}

// Value v of lane l (l wave-uniform), in scalar registers.
__device__ __forceinline__ int64_t lane64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(uint64_t(v)), l);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(uint64_t(v) >> 32), l);
  return int64_t((uint64_t(hi) << 32) | lo);
}

// Lengths (and, with several queries per sequence, the first packed row and the query
// count) of the first kSeqCache sequences, one per lane and 64-sequence chunk, with the
// inclusive running sum of their segment units.  A wave loads them once, every load
// issued before any is used; the share's location and each later segment's geometry
// then come from registers (readlane) instead of a chain of dependent loads.  Sequences
// past them are read from memory.
constexpr int kSeqChunks = 4;
constexpr int kSeqCache = 64 * kSeqChunks;

template <bool MQ>
struct SeqCache {
  int L[kSeqChunks];
  int q0[MQ ? kSeqChunks : 1], nq[MQ ? kSeqChunks : 1];
  int64_t incl[kSeqChunks];  // segment units (per kv head) of sequences 0 .. 64k + lane
  int64_t run;               // ... of all cached sequences
  int n;                     // cached sequences: min(S, kSeqCache)
};

// Entry s (< kSeqCache, wave-uniform) of a cached array: lane s mod 64 of chunk s / 64.
// Every chunk is read with a constant index (a run-time index into the array would
// put the cache in scratch memory).
__device__ __forceinline__ int cached(const int (&v)[kSeqChunks], int s) {
  const int l = s & 63, k = s >> 6;
  int r = __builtin_amdgcn_readlane(v[0], l);
#pragma unroll
  for (int j = 1; j < kSeqChunks; ++j) {
    const int x = __builtin_amdgcn_readlane(v[j], l);
    r = k == j ? x : r;
  }
  return r;
}

template <bool MQ, int SC>
__device__ __forceinline__ void load_seqs(SeqCache<MQ>& c, const int32_t* __restrict__ lens,
                                          const int32_t* __restrict__ cu, int W, int S, int lane) {
  c.n = min(S, kSeqCache);
#pragma unroll
  for (int k = 0; k < kSeqChunks; ++k) {
    const int s = min(64 * k + lane, S - 1);  // unconditional loads; lanes past S unused
    c.L[k] = lens[s];
    if constexpr (MQ) {
      c.q0[k] = cu[s];
      c.nq[k] = cu[s + 1];
    }
  }
  int64_t run = 0;
#pragma unroll
  for (int k = 0; k < kSeqChunks; ++k) {
    if constexpr (MQ) c.nq[k] -= c.q0[k];
    if (64 * k < c.n) {  // wave-uniform
      const int64_t nu = 64 * k + lane < c.n ? int64_t(seg_units<SC>(c.L[k], MQ ? c.nq[k] : 1, W)) : 0;
      c.incl[k] = run + wave_incl_scan(nu, lane);
      run = lane64(c.incl[k], 63);
    } else {
      c.incl[k] = run;
    }
  }
  c.run = run;
}

// Length, first packed row and query count of sequence s (wave-uniform).
template <bool MQ>
__device__ __forceinline__ void seq_info(const SeqCache<MQ>& c, const int32_t* __restrict__ lens,
                                         const int32_t* __restrict__ cu, int s, int& L, int& q0, int& nq) {
  if (s < c.n) {
    L = cached(c.L, s);
    if constexpr (MQ) {
      q0 = cached(c.q0, s);
      nq = cached(c.nq, s);
    }
  } else {
    L = uniform32(lens[s]);
    if constexpr (MQ) {
      q0 = uniform32(cu[s]);
      nq = uniform32(cu[s + 1]) - q0;
    }
  }
  if constexpr (!MQ) {
    q0 = s;
    nq = 1;
  }
}

// Total units of all (sequence, kv head) segments.
template <bool MQ, int SC>
__device__ __forceinline__ int64_t total_blocks(const SeqCache<MQ>& c, const int32_t* __restrict__ lens,
                                                const int32_t* __restrict__ cu, int W, int S, int Hkv,
                                                int lane) {
  int64_t sum = 0;
  if (S > kSeqCache) {  // wave-uniform
    for (int s = kSeqCache + lane; s < S; s += 64) sum += seg_units<SC>(lens[s], queries_of(cu, s), W);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  }
  return uniform64((c.run + sum) * Hkv);
}

// Sequence whose segments contain flat unit f, and its cum (units before it).
template <bool MQ, int SC>
__device__ __forceinline__ void locate(const SeqCache<MQ>& c, const int32_t* __restrict__ lens,
                                       const int32_t* __restrict__ cu, int W, int S, int Hkv, int64_t f,
                                       int lane, int& s_out, int64_t& cum_out) {
  if (f < Hkv * c.run) {
    // first chunk k with a sequence whose segments reach past f, and that sequence's
    // lane; every chunk is read with a constant index (a run-time one would put the
    // cache in memory)
    int k = 0;
    uint64_t hit = 0;
#pragma unroll
    for (int j = kSeqChunks - 1; j >= 0; --j) {
      const uint64_t h = __ballot(64 * j + lane < c.n && Hkv * c.incl[j] > f);
      if (h) {
        k = j;
        hit = h;
      }
    }
    const int first = __builtin_ctzll(hit);
    int64_t incl = lane64(c.incl[0], first);
#pragma unroll
    for (int j = 1; j < kSeqChunks; ++j) {
      const int64_t x = lane64(c.incl[j], first);
      incl = k == j ? x : incl;
    }
    int L, q0, nq;
    s_out = 64 * k + first;
    seq_info(c, lens, cu, s_out, L, q0, nq);
    cum_out = incl - seg_units<SC>(L, nq, W);
    return;
  }
  int64_t run = c.run;
  for (int base = kSeqCache; base < S; base += 64) {
    const int s = base + lane;
    const int64_t nu = s < S ? int64_t(seg_units<SC>(lens[s], queries_of(cu, s), W)) : 0;
    const int64_t incl = wave_incl_scan(nu, lane);
    const uint64_t hit = __ballot(s < S && Hkv * (run + incl) > f);
    if (hit) {
      const int first = __builtin_ctzll(hit);
      s_out = base + first;
      cum_out = uniform64(run + __shfl(incl - nu, first, 64));
      return;
    }
    run = uniform64(run + __shfl(incl, 63, 64));
  }
  s_out = S;
  cum_out = run;
}

// MQ (several queries per sequence: prefill chunks of at most 16 / G queries): the
// tile's rows are (query, head) pairs, query j of sequence s is packed row
// cu_q_lens[s] + j at position L - nq + j, and records hold 16 rows.  Otherwise one
// query per sequence (packed row s) and records of G rows.
template <int KV, int D, int G, bool SMALLP, bool MQ, bool DENSE = false>
__global__ __launch_bounds__(64 * kWgWaves) __attribute__((amdgpu_waves_per_eu(kAutoWavesPerEu<KV, DENSE>, kAutoWavesPerEu<KV, DENSE>))) void decode_auto_kernel(AttnArgs a) {
  static_assert(!DENSE || (KV == DT_FP8 && !SMALLP && !MQ), "dense decode: one-query FP8 calls, pages >= 32");
  if (halted(a.cache)) return;
  constexpr int ROWS = MQ ? 16 : G;
  const int lane = threadIdx.x & 63;
  // Workgroups go to the eight XCDs round robin (workgroup b to XCD b mod 8).  With one
  // query per sequence, XCD x takes the x-th eighth of the share order, so each L2 serves
  // a contiguous run of sequences: pages that neighbouring requests share (a common
  // prefix) and their table rows are fetched into one L2 instead of all eight (FP8
  // shared-prefix batch 209 -> 199 us; the other decode batches within +-1 %).  Calls
  // with several queries per sequence measured 2 % slower with it and keep the
  // identity order.
  const int nwg = gridDim.x;
  const int bx = (!MQ && nwg % kXcds == 0) ? (blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds : blockIdx.x;
  const int w = bx * kWgWaves + uniform32(threadIdx.x >> 6);
  if (w >= a.num_waves) return;
  const int S = a.seqs.num_seqs, Hkv = a.cache.num_kv_heads;
  const int32_t* lens = a.seqs.context_lens;
  const int32_t* cu = MQ ? a.cu_q_lens : nullptr;
  const int W = a.seqs.window;
  SeqCache<MQ> sc;
  constexpr int SC = kSegCost<KV, DENSE>;
  load_seqs<MQ, SC>(sc, lens, cu, W, S, lane);
  const int64_t T = total_blocks<MQ, SC>(sc, lens, cu, W, S, Hkv, lane);
  // (a share of more than SC units holds at least one block)
  const int64_t share = max(int64_t(max(a.min_share, SC + 1)), (T + a.num_waves - 1) / a.num_waves);
  const int64_t f0 = int64_t(w) * share;
  int4* desc = a.ws_desc + w;
  if (f0 >= T) {
    if (lane == 0) *desc = make_int4(-1, 0, 0, 0);
    return;
  }
  const int64_t fend = min(T, f0 + share);
  int s;
  int64_t cum;
  locate<MQ, SC>(sc, lens, cu, W, S, Hkv, f0, lane, s, cum);
  const int64_t tile_b = tile_bytes(KV, a.cache.page_size, D);
  const int log2P = a.cache.log2_page;
  // The piece of this wave's share in segment (s, g) that holds flat unit f: its
  // sequence geometry, the unit gs of the segment's first block, and the unit fs of the
  // piece's first block (f, or gs when f lies in the segment's start cost).
  struct Piece {
    int L, q0, nq, blo, nb, g;
    int64_t gs, fs;
  };
  auto piece_of = [&](int s_, int64_t cum_, int64_t f_) {
    Piece pc;
    seq_info(sc, lens, cu, s_, pc.L, pc.q0, pc.nq);
    pc.nb = seg_blocks(pc.L, pc.nq, W, pc.blo);
    const int nu = pc.nb + SC;
    const int64_t seg0 = Hkv * cum_;
    pc.g = int((f_ - seg0) / nu);
    pc.gs = seg0 + int64_t(pc.g) * nu + SC;
    pc.fs = max(f_, pc.gs);
    return pc;
  };
  // the sequence and cum of the segment after pc's
  auto advance = [&](int& s_, int64_t& cum_, const Piece& pc) {
    if (pc.g + 1 == Hkv) {
      cum_ += pc.nb + SC;
      ++s_;
    }
  };
  // Block-table window of the piece's first page (pages of >= 32 tokens), loaded one
  // piece ahead: a wave that moves to its next segment then waits only for that
  // segment's first blocks, not for the table entries in front of them.
  auto window_of = [&](int s_, const Piece& pc) {
    PageWindow win{0, 0};
    if constexpr (!SMALLP) {
      const int first_blk = pc.blo + int(pc.fs - pc.gs);
      load_window(win, a.seqs.block_tables + int64_t(s_) * a.seqs.max_pages_per_seq,
                  first_blk >> (log2P - LOG2_BT), (pc.L + (1 << log2P) - 1) >> log2P, lane);
    }
    return win;
  };
  // Fold the piece of segment (s, g) from its first block to the segment's end or fend.
  // `first`: the share's first piece (record slot 0, described to the merge).
  auto run_piece = [&](int s_, const Piece& pc, bool first, const PageWindow& win) {
    const int b0 = int(pc.fs - pc.gs);
    const int b1 = int(min(int64_t(pc.nb), fend - pc.gs));
    if (first && lane == 0) {
      // This wave merges its first segment when that segment started in an earlier
      // wave (w0: the one whose share holds its first block) and ends inside this one.
      // Record slot of w0: 0 if the segment is w0's first (w0's share starts at or
      // after the segment's first unit), else 1.
      const int64_t w0 = pc.gs / share;
      const bool merges = pc.gs < f0 && pc.gs + pc.nb <= fend;
      *desc = make_int4(s_, pc.g, int(w0), merges ? (1 | (pc.gs - SC > w0 * share ? 2 : 0)) : 0);
    }
    float qk_scale, vscale;
    scales<KV>(a, pc.g, qk_scale, vscale);
    bf16x8 qf[D / 32];
    load_q<D, G>(qf, a.q, pc.q0, pc.nq, a.num_q_heads, pc.g, lane);
    State<D> st;
    state_init(st);
    const int32_t* bt = a.seqs.block_tables + int64_t(s_) * a.seqs.max_pages_per_seq;
    const int L = pc.L, nq = pc.nq;
    const int t_end = min(L, (pc.blo + b1) << LOG2_BT);
    const int pos = L - nq + (lane & 15) / G;  // position of this lane's row's query
    const RowKeys k{t_end, pos + 1, min(t_end, L - nq + 1), window_lo(pos, W), window_lo(L - 1, W)};
    run_range<KV, D, SMALLP, DENSE>(st, qf, qk_scale, static_cast<const char*>(a.cache.pool), bt, pc.blo + b0,
                                    pc.blo + b1, k, L, log2P, Hkv * tile_b, pc.g * tile_b, lane, &win);
    const bool complete = b0 == 0 && b1 == pc.nb;
    finish<D, G, ROWS>(st, a, pc.q0, nq, pc.g, complete, int64_t(w) * 2 + (first ? 0 : 1), qk_scale, vscale,
                       lane);
  };
  // Order of the pieces: a share whose first piece continues a segment begun in an
  // earlier wave folds that piece last, so every wave starts at the head of a segment.
  // The heads of neighbouring requests' segments are where a shared prefix lies: the
  // waves that read the same prefix pages then read them at about the same time, and
  // one L2 fetch serves several of them.  Each piece is computed exactly as in flat
  // order (same blocks, same record slots), so the results do not change.  A share
  // starting in a segment's start cost begins at that segment's first block; one ending
  // there holds none of that segment.
  const int s_first = s;
  const Piece p_first = piece_of(s, cum, f0);
  int cs = s;
  int64_t ccum = cum;
  advance(cs, ccum, p_first);
  Piece cp = p_first;
  bool later = p_first.gs + p_first.nb < fend;  // a piece after the first one holds blocks
  if (later) {
    cp = piece_of(cs, ccum, p_first.gs + p_first.nb);
    later = cp.fs < fend;
  }
  const bool defer = f0 > p_first.gs && later;
  bool tail = defer;  // the first piece still to be folded after the others
  bool cfirst = true, clast = !later;
  if (defer) {
    cfirst = false;
  } else {
    cs = s;
    ccum = cum;
    cp = p_first;
  }
  PageWindow cw = window_of(cs, cp);
  for (;;) {
    // the piece after this one, and its window, before this one is folded
    int ns = cs;
    int64_t ncum = ccum;
    advance(ns, ncum, cp);
    const int64_t nf = cp.gs + min(int64_t(cp.nb), fend - cp.gs);
    bool has_next = !clast, nfirst = false, nlast = false;
    Piece np = cp;
    if (has_next) {
      bool flat = nf < fend;  // the next piece in flat order, if it holds blocks
      if (flat) {
        np = piece_of(ns, ncum, nf);
        flat = np.fs < fend;
      }
      if (!flat) {
        if (tail) {
          ns = s_first;
          np = p_first;
          nfirst = nlast = true;
          tail = false;
        } else {
          has_next = false;
        }
      }
    }
    PageWindow nw{0, 0};
    if (has_next) nw = window_of(ns, np);
    run_piece(cs, cp, cfirst, cw);
    if (!has_next) break;
    cs = ns;
    ccum = ncum;
    cp = np;
    cfirst = nfirst;
    clast = nlast;
    cw = nw;
  }
}

// Merge of one cut (sequence, kv head) segment of the balanced schedule, by the
// workgroup of the wave that holds its last piece (a wave is the last one of at most
// one cut segment: its first).  The pieces are in waves w0 .. w; the record of wave v
// is slot 0, except slot 1 for w0 when the segment is not w0's first.  One workgroup
// per wave (most find nothing to do and exit at once): a loop over several
// descriptors per workgroup would chain their dependent loads.  The call is bound by
// the launch and the two dependent loads (descriptor, then records): one wave per
// descriptor, 128 threads (no LDS combine), or records touched before the descriptor
// arrives all measured equal or slower.
#ifndef PKV_AUTO_MERGE_THREADS
#define PKV_AUTO_MERGE_THREADS 256
#endif
constexpr int kAutoMergeThreads = PKV_AUTO_MERGE_THREADS;

template <int D, int G, bool MQ>
__global__ __launch_bounds__(kAutoMergeThreads) void merge_auto_kernel(AttnArgs a) {
  if (halted(a.cache)) return;
  const int w = blockIdx.x;
  const int4 d = a.ws_desc[w];  // (sequence, kv head, w0, flags)
  if (d.x < 0 || !(d.w & 1)) return;
  const int w0 = d.z;
  const bool slot1 = d.w & 2;
  const int q0 = MQ ? a.cu_q_lens[d.x] : d.x;
  const int nq = MQ ? a.cu_q_lens[d.x + 1] - q0 : 1;
  merge_partials<D, G, MQ ? 16 : G, kAutoMergeThreads>(a, q0, nq, d.y, w - w0 + 1, [w0, slot1](int i) {
    return int64_t(w0 + i) * 2 + ((i == 0 && slot1) ? 1 : 0);
  });
}

// Merge of the fixed partitions of one (sequence, kv head).
template <int D, int G>
__global__ __launch_bounds__(kMergeThreads) void merge_fixed_kernel(AttnArgs a) {
  if (halted(a.cache)) return;
  const int sg = blockIdx.x;
  const int Hkv = a.cache.num_kv_heads;
  const int g = sg % Hkv, s = sg / Hkv;
  const int n = (a.seqs.context_lens[s] + a.chunk - 1) / a.chunk;
  if (n <= 1) return;  // written directly
  const int64_t r0 = int64_t(sg) * a.max_splits;
  merge_partials<D, G, G, kMergeThreads>(a, s, 1, g, n, [r0](int i) { return r0 + i; });
}

// ---- host side ---------------------------------------------------------------------------

template <int KV, int D, int G, bool SMALLP>
hipError_t launch_t(const AttnArgs& a, const MfmaPlan& p, hipStream_t st) {
  if (p.auto_mode) {
    const dim3 grid(unsigned((p.waves + kWgWaves - 1) / kWgWaves)), block(64 * kWgWaves);
    if (p.multi_query) {
      if constexpr (G <= 8) {  // 16 / G >= 2 queries per tile
        hipLaunchKernelGGL((decode_auto_kernel<KV, D, G, SMALLP, true>), grid, block, 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((merge_auto_kernel<D, G, true>), dim3(p.waves), dim3(kAutoMergeThreads), 0, st, a);
        return hipGetLastError();
      }
      return hipErrorInvalidValue;
    }
    if constexpr (KV == DT_FP8 && !SMALLP) {
      if (p.dense)
        hipLaunchKernelGGL((decode_auto_kernel<KV, D, G, false, false, true>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((decode_auto_kernel<KV, D, G, false, false>), grid, block, 0, st, a);
    } else {
      if (p.dense) return hipErrorInvalidValue;
      hipLaunchKernelGGL((decode_auto_kernel<KV, D, G, SMALLP, false>), grid, block, 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((merge_auto_kernel<D, G, false>), dim3(p.waves), dim3(kAutoMergeThreads), 0, st, a);
    return hipGetLastError();
  }
  const int64_t nblk = int64_t(a.seqs.num_seqs) * a.cache.num_kv_heads * a.max_splits;
  hipLaunchKernelGGL((decode_fixed_kernel<KV, D, G, SMALLP>), dim3(unsigned((nblk + kWgWaves - 1) / kWgWaves)),
                     dim3(64 * kWgWaves), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL((merge_fixed_kernel<D, G>), dim3(unsigned(int64_t(a.seqs.num_seqs) * a.cache.num_kv_heads)),
                     dim3(kMergeThreads), 0, st, a);
  return hipGetLastError();
}

template <int KV, int D, int G>
hipError_t dispatch_p(const AttnArgs& a, const MfmaPlan& p, hipStream_t st) {
  if constexpr (KV == DT_MXFP4) {  // MXFP4 tiles need pages of >= 32 tokens
    return a.cache.page_size >= BT ? launch_t<KV, D, G, false>(a, p, st) : hipErrorInvalidValue;
  } else {
    return a.cache.page_size >= BT ? launch_t<KV, D, G, false>(a, p, st) : launch_t<KV, D, G, true>(a, p, st);
  }
}

template <int KV, int D>
hipError_t dispatch_g(const AttnArgs& a, const MfmaPlan& p, hipStream_t st) {
  switch (a.num_q_heads / a.cache.num_kv_heads) {
    case 1: return dispatch_p<KV, D, 1>(a, p, st);
    case 2: return dispatch_p<KV, D, 2>(a, p, st);
    case 4: return dispatch_p<KV, D, 4>(a, p, st);
    case 8: return dispatch_p<KV, D, 8>(a, p, st);
    case 16: return dispatch_p<KV, D, 16>(a, p, st);
  }
  return hipErrorInvalidValue;
}

template <int KV>
hipError_t dispatch_d(const AttnArgs& a, const MfmaPlan& p, hipStream_t st) {
  return a.cache.head_dim == 64 ? dispatch_g<KV, 64>(a, p, st) : dispatch_g<KV, 128>(a, p, st);
}

// Kernel whose occupancy sizes the auto grid (one instance per head_dim / dtype is
// representative: G only changes which MFMA rows are used).
template <int KV, int D>
const void* auto_kernel_for(int G, bool smallp, bool dense) {
  // (MXFP4 has no short-page kernels: its instance stands in for both)
#define PKV_K(GG) (smallp ? reinterpret_cast<const void*>(&decode_auto_kernel<KV, D, GG, KV != DT_MXFP4, false>)   \
                   : dense && KV == DT_FP8                                                                       \
                       ? reinterpret_cast<const void*>(&decode_auto_kernel<DT_FP8, D, GG, false, false, true>)   \
                       : reinterpret_cast<const void*>(&decode_auto_kernel<KV, D, GG, false, false>))
  switch (G) {
    case 1: return PKV_K(1);
    case 2: return PKV_K(2);
    case 4: return PKV_K(4);
    case 8: return PKV_K(8);
    default: return PKV_K(16);
  }
#undef PKV_K
}

}  // namespace

bool mfma_decode_supported(int kv_dtype, int q_dtype, int head_dim, int group, int page_size) {
  return (kv_dtype == DT_BF16 || kv_dtype == DT_FP8 || kv_dtype == DT_MXFP4) && q_dtype == DT_BF16 &&
         (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16) &&
         page_size >= (kv_dtype == DT_MXFP4 ? BT : 8);
}

int mfma_auto_waves(int kv_dtype, int head_dim, int group, int page_size, bool dense) {
  const bool smallp = page_size < BT;
  dense = dense && kv_dtype == DT_FP8 && !smallp;
  const void* k = kv_dtype == DT_BF16
                      ? (head_dim == 64 ? auto_kernel_for<DT_BF16, 64>(group, smallp, false)
                                        : auto_kernel_for<DT_BF16, 128>(group, smallp, false))
                  : kv_dtype == DT_FP8
                      ? (head_dim == 64 ? auto_kernel_for<DT_FP8, 64>(group, smallp, dense)
                                        : auto_kernel_for<DT_FP8, 128>(group, smallp, dense))
                      : (head_dim == 64 ? auto_kernel_for<DT_MXFP4, 64>(group, false, false)
                                        : auto_kernel_for<DT_MXFP4, 128>(group, false, false));
  return resident_blocks(k, 64 * kWgWaves) * kWgWaves;
}

hipError_t launch_mfma_decode(const AttnArgs& a, const MfmaPlan& p, hipStream_t st) {
  if (a.seqs.num_seqs == 0) return hipSuccess;
  switch (a.cache.dtype) {
    case DT_BF16: return dispatch_d<DT_BF16>(a, p, st);
    case DT_FP8: return dispatch_d<DT_FP8>(a, p, st);
    case DT_MXFP4: return dispatch_d<DT_MXFP4>(a, p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
