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
// loads as decode) feeds kPrefillTiles x 16 rows.  This per-wave kernel serves pages of
// fewer than 32 tokens and, on any page size, chunks that at most two waves' tiles
// cover (mfma_prefill_geometry); other prefill runs on the LDS-shared kernel below.
// Causality is a per-row key limit, applied only on the blocks that reach a row's
// position.
//
// Work item (one wave): (sequence, kv head, key split, query tile).  When the chunk
// alone does not give enough waves to fill the device, each tile's key range is cut
// into equal block ranges (splits), whose normalised partials and log-sum-exps are
// merged exactly by a second kernel.  Workgroups go to the XCDs round robin; the
// grid is ordered so that all query tiles of one (sequence, kv head, split) land on
// the same XCD and read the same K/V blocks through its L2.
#include "stage.h"

namespace pkv {
namespace {

// 16-row tiles per wave of the per-wave kernel: four for D = 64; two for D = 128, where
// four tiles' accumulators, queries and two blocks in flight exceed the 256 vector
// registers a wave can address and spill.
template <int D>
constexpr int kPrefillTiles = D == 128 ? 2 : 4;

// Query tile geometry for G query heads per kv head (per-wave kernel: D's tile count).
template <int G, int D = 64>
struct PfGeom {
  static constexpr int QPT = 16 / G;                    // queries per 16-row tile
  static constexpr int QW = kPrefillTiles<D> * QPT;     // queries per wave
};

// Finish the NT row tiles of a wave: rows of the chunk only.  One split: output and
// log-sum-exp; several: partial record (row, kv head, split) for the merge kernel.
// lsum: NULL, or each tile's sums of the weights in the O layout (lane (n, c) holds those
// of rows 4c .. 4c+3, in every column n), summed on the matrix cores; else st[r].l holds
// the lane's share of its row's sum.
template <int D, int G, int NT>
__device__ __forceinline__ void prefill_finish(const AttnArgs& a, const State<D> (&st)[NT], int q0, int C,
                                               int cq0, int g, int split, float qk_scale, float vscale,
                                               int lane, const f32x4* lsum = nullptr) {
  constexpr int QPT = PfGeom<G>::QPT;
  const int n = lane & 15, c = lane >> 4;
  const int Hkv = a.cache.num_kv_heads, Hq = a.num_q_heads, nsplit = a.max_splits;
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    float l, inv[4];
    if (lsum) {
      // row n's sum sits in lane (any column, n >> 2), element n & 3
      const int i = n & 3;
      const float mine = i == 0 ? lsum[r][0] : i == 1 ? lsum[r][1] : i == 2 ? lsum[r][2] : lsum[r][3];
      l = __shfl(mine, 16 * (n >> 2) + n, 64);
#pragma unroll
      for (int k = 0; k < 4; ++k) inv[k] = lsum[r][k] > 0.f ? vscale / lsum[r][k] : 0.f;
    } else {
      l = st[r].l;
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lr = __shfl(l, 4 * c + k, 64);
        inv[k] = lr > 0.f ? vscale / lr : 0.f;
      }
    }
    const float lse = row_lse(st[r].m, l, qk_scale);  // row n
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

template <int KV, int D, int G, bool SMALLP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_kernel(AttnArgs a) {
  if (halted(a.cache)) return;
  constexpr int NT = kPrefillTiles<D>, QPT = PfGeom<G, D>::QPT, QW = PfGeom<G, D>::QW;
  const int lane = threadIdx.x, n = lane & 15, c = lane >> 4;
  const int Hkv = a.cache.num_kv_heads, Hq = a.num_q_heads, nsplit = a.max_splits;
  const int QT = a.pf_qtiles;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int grp = xcd + kXcds * (slot / QT), qt = slot % QT;
  if (grp >= a.seqs.num_seqs * Hkv * nsplit) return;
  const int split = grp % nsplit, sg = grp / nsplit;
  const int g = sg % Hkv, s = sg / Hkv;
  const int cq0 = uniform32(a.cu_q_lens[s]), C = uniform32(a.cu_q_lens[s + 1]) - cq0;
  const int q0 = qt * QW;
  if (q0 >= C) return;
  const int L = uniform32(a.seqs.context_lens[s]);
  const int W = a.seqs.window;
  const int pos0 = L - C;                          // position of query 0 of the chunk
  const int kend = pos0 + min(C, q0 + QW);         // keys [0, kend) reach this tile
  const int nb = (kend + BT - 1) >> LOG2_BT;
  const int blo = window_lo(pos0 + q0, W) >> LOG2_BT;  // blocks before the first query's window: none
  const int b0 = blo + int(int64_t(nb - blo) * split / nsplit);
  const int b1 = blo + int(int64_t(nb - blo) * (split + 1) / nsplit);

  float qk_scale, vscale;
  scales<KV>(a, g, qk_scale, vscale);
  // Q^T operands and key limits: lane (n, c) of tile r is row n = query q0 + r*QPT +
  // n/G, head g*G + n%G; it sees keys t < lim[r] (0 for rows past the chunk).
  bf16x8 qf[NT][D / 32];
  int lim[NT], lo[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const int qi = q0 + r * QPT + n / G;
    lim[r] = qi < C ? pos0 + qi + 1 : 0;
    lo[r] = window_lo(pos0 + qi, W);
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
  const int lo_max = window_lo(pos0 + min(C, q0 + QW) - 1, W);  // largest window start of its live rows
  State<D> st[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) state_init(st[r]);

  if (b0 < b1) {
    const int64_t tile_b = tile_bytes(KV, a.cache.page_size, D);
    const int32_t* bt = a.seqs.block_tables + int64_t(s) * a.seqs.max_pages_per_seq;
    run_blocks<KV, D, SMALLP>(
        static_cast<const char*>(a.cache.pool), bt, b0, b1, L, a.cache.log2_page, Hkv * tile_b,
        g * tile_b, lane, [&](auto& blk, int t) {
          if (t + BT > L) mask_v_tail<D>(blk, L - t, lane);
          const auto& rb = ready<D>(blk);  // an MXFP4 block decoded once for all tiles
#pragma unroll
          for (int r = 0; r < NT; ++r) {
            float sc[8];
            block_scores<D>(rb, qf[r], sc);
            if (t + BT > lim_min || t < lo_max) {  // wave-uniform: reaches a row's position or window start
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int tk = t + tok_of(c, e);
                if (tk >= lim[r] || tk < lo[r]) sc[e] = -INFINITY;
              }
            }
            softmax_pv<D>(st[r], rb, sc, qk_scale, lane);
          }
        });
  }

  prefill_finish<D, G, NT>(a, st, q0, C, cq0, g, split, qk_scale, vscale, lane);
}

// ---- LDS-shared variant (pages of >= 32 tokens) -----------------------------------------
// A workgroup of kPfWaves waves (one per SIMD, kPfTiles row tiles each) shares one K/V
// stream: every 32-token block is fetched once per workgroup -- each thread loads its
// 16-byte pieces of it into registers five blocks ahead (two register slots), then
// writes them into one of five LDS stages three blocks ahead -- and each wave reads its
// MFMA operands from the stage with the same lane offsets as from the tile in HBM.  The
// stage layout mirrors the block's HBM layout, in bf16: K as D/32 chunks of [32 tokens]
// [32 dims], then V as [D][32 positions].  FP8 and MXFP4 blocks are decoded to bf16 as
// they are staged, once per workgroup rather than once per wave that reads them (twice
// the LDS bytes of an FP8 stage, a sixth of the conversions).  A wave computes the scores
// of block i+1 (matrix cores) while it runs the softmax of block i (vector ALU) and then
// the P.V products of block i: the two units work at once within each wave, instead
// of every wave waiting on one then the other between barriers.  Five stages let one
// barrier serve two blocks: during a pair of steps the waves read the stages of three
// blocks and write those of the next two (with three stages, one barrier per block:
// 1 - 2 % slower on the mixed batch's prefill calls).
#ifndef PKV_PF_TILES
#define PKV_PF_TILES 2
#endif
constexpr int kPfTiles = PKV_PF_TILES;   // 16-row tiles per wave of the LDS-shared kernel
constexpr int kPfStages = 5;             // LDS stages of 32-token blocks (bf16)
#ifndef PKV_PF_SCHED
#define PKV_PF_SCHED 2  // vector instructions the scheduler puts after each MFMA of a step (0: its own order)
#endif
// Per cache type: MXFP4 steps keep the scheduler's own order (its decoding conversions
// already sit between the matrix instructions; with the interleave hint its prefill call
// measured 191 against 186.5 us), bf16 and FP8 take the hint (equal or 1 % faster).
template <int KV>
constexpr int kPfSched = KV == DT_MXFP4 ? 0 : PKV_PF_SCHED;

// Workgroup barrier; LDS writes and reads of this wave are complete before it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int KV, int D, int G>
__global__ __launch_bounds__(64 * kPfWaves) __attribute__((amdgpu_waves_per_eu(kPfWaves / 4, kPfWaves / 4))) void prefill_lds_kernel(AttnArgs a) {
  if (halted(a.cache)) return;
  using SL = Stager<KV, D, kPfThreads>;
  constexpr int NT = kPfTiles, QPT = PfGeom<G>::QPT, QWV = NT * QPT;
  constexpr int QWG = kPfWaves * QWV;
  __shared__ __attribute__((aligned(1024))) char smem[kPfStages * SL::BYTES];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, c = lane >> 4;
  const int Hkv = a.cache.num_kv_heads, Hq = a.num_q_heads, nsplit = a.max_splits;
  const int QT = a.pf_qtiles;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int grp = xcd + kXcds * (slot / QT), qt = slot % QT;
  if (grp >= a.seqs.num_seqs * Hkv * nsplit) return;  // whole workgroup
  const int split = grp % nsplit, sg = grp / nsplit;
  const int g = sg % Hkv, s = sg / Hkv;
  const int cq0 = uniform32(a.cu_q_lens[s]), C = uniform32(a.cu_q_lens[s + 1]) - cq0;
  if (qt * QWG >= C) return;                            // whole workgroup
  const int L = uniform32(a.seqs.context_lens[s]);
  const int W = a.seqs.window;
  const int pos0 = L - C;
  const int kend = pos0 + min(C, qt * QWG + QWG);       // keys any row of the group sees
  const int nb = (kend + BT - 1) >> LOG2_BT;
  const int blo = window_lo(pos0 + qt * QWG, W) >> LOG2_BT;  // blocks before the first query's window: none
  const int b0 = blo + int(int64_t(nb - blo) * split / nsplit);
  const int b1 = blo + int(int64_t(nb - blo) * (split + 1) / nsplit);
  const int q0 = qt * QWG + w * QWV;                    // this wave's first query
  const bool live = q0 < C;

  float qk_scale, vscale;
  scales<KV>(a, g, qk_scale, vscale);
  bf16x8 qf[NT][D / 32];
  int lim[NT], lo[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const int qi = q0 + r * QPT + n / G;
    lim[r] = qi < C ? pos0 + qi + 1 : 0;
    lo[r] = window_lo(pos0 + qi, W);
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
  const int lim_min = pos0 + q0 + 1;
  const int lo_max = live ? window_lo(pos0 + min(C, q0 + QWV) - 1, W) : 0;  // largest window start of its rows
  State<D> st[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) state_init(st[r]);
  // Row sums of the weights in the O layout, accumulated on the matrix cores as P . 1 (one
  // more product per tile and block) instead of 8 vector adds per tile and block: the
  // vector ALU, not the matrix cores, is the busier unit here.  They sum the bf16 weights
  // the P.V product uses.
  f32x4 lsum[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) lsum[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  Frag8 onesf;
  onesf.q = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);  // bf16 1.0 x 8
  const bf16x8 ones = onesf.v;

  const int log2P = a.cache.log2_page, P = 1 << log2P;
  const int64_t tile_b = tile_bytes(KV, P, D);
  const BlockSrc src{static_cast<const char*>(a.cache.pool), a.seqs.block_tables + int64_t(s) * a.seqs.max_pages_per_seq,
                     log2P, Hkv * tile_b, g * tile_b};
  auto fetch_any = [&](typename SL::Regs& r, int blk) { SL::fetch(r, src, blk, tid); };
  auto stash_any = [&](typename SL::Regs& r, int stage, int blk) {
    SL::stash(r, smem + stage * SL::BYTES, L - (blk << LOG2_BT), tid);
  };

  const int nblk = b1 - b0;
  // lane offset of the operand load in a K chunk / V tile (row n, segment c)
  const uint32_t lk = stage_lane_offset(lane);
  // Raw scores of block b0+i (stage i%5) for the wave's tiles.
  auto scores = [&](int i, float (&sc)[NT][8]) {
    const char* stg = smem + (i % kPfStages) * SL::BYTES;
    Block<D> b;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      b.ka[j] = SL::k_operand(stg, j, 0, lk);
      b.kb[j] = SL::k_operand(stg, j, 1, lk);
    }
#pragma unroll
    for (int r = 0; r < NT; ++r) block_scores<D>(b, qf[r], sc[r]);
  };
  // Step i: block i+3 goes from its register slot into stage (i+3)%5 -- that of block
  // i-2, last read before the most recent barrier -- and the slot refills with block
  // i+5 (clamped to the last block: a harmless repeat near the end).  The barrier comes
  // after every odd step: within a pair of steps (2j, 2j+1) the waves read the stages of
  // blocks 2j .. 2j+2 and write those of 2j+3 and 2j+4, five distinct stages.  The
  // scores of block i+1 go into nxt (stage (i+1)%5, written two steps or more before,
  // with a barrier since; clamped at the end).  Then block i is folded: its scores (cur, from the previous step) are
  // masked where the block reaches a row's position or lies past the wave's rows
  // (every weight there is 0, so such a block changes nothing), maxima and the rare
  // rescale vote come first, then the exponentials and P.V products of block i, which
  // the scheduler interleaves.  Where the scores of block i+1 are issued decides what
  // their matrix instructions overlap: first in the step, before the staging, they run
  // under its LDS writes (and the MXFP4 decoding conversions).  Measured on the mixed
  // batch's prefill call, against issuing them after the staging, before the maxima:
  // bf16 165.0 against 169.8 us, FP8 172.7 against 173.5, MXFP4 182.9 against 186.4.
  // (With one barrier per block the bf16 and FP8 calls had been faster the other way.)
  const int last = b1 - 1;
  typename SL::Regs ra, rb;
  float sa_[NT][8], sb_[NT][8];
  auto step = [&](auto& rs, int i, float (&cur)[NT][8], float (&nxt)[NT][8]) {
    const int t = (b0 + i) << LOG2_BT;
    const int blk3 = min(b0 + i + 3, last);
    if (live) scores(min(i + 1, nblk - 1), nxt);
    stash_any(rs, (i + 3) % kPfStages, blk3);
    fetch_any(rs, min(b0 + i + 5, last));
    // a wave whose rows all lie past the chunk (short chunks) only stages its share
    if (live) {
    if (t + BT > lim_min || t < lo_max) {  // wave-uniform: reaches a row's position or window start
#pragma unroll
      for (int r = 0; r < NT; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tk = t + tok_of(c, e);
          if (tk >= lim[r] || tk < lo[r]) cur[r][e] = -INFINITY;
        }
    }
    float off[NT];
    softmax_head<D, NT>(st, cur, qk_scale, off, lane, lsum);
    const char* stg = smem + (i % kPfStages) * SL::BYTES;
    bf16x8 vv[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) vv[dt] = SL::v_operand(stg, dt, lk);
    Frag8 pa[NT];
    softmax_tail<NT, false>(st, cur, qk_scale, off, pa);
#pragma unroll
    for (int r = 0; r < NT; ++r) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) st[r].o[dt] = mma(pa[r].v, vv[dt], st[r].o[dt]);
      lsum[r] = mma(pa[r].v, ones, lsum[r]);  // the weights' row sums: P . 1 (one product per tile)
    }
    if constexpr (kPfSched<KV> > 0) {
      // exponentials and conversions of block i around the scores of block i+1
#pragma unroll
      for (int k = 0; k < NT * D / 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x0002, kPfSched<KV>, 0);  // vector ALU
      }
    }
    }
    if (i & 1) stage_barrier();  // one barrier per two blocks
  };
  if (nblk > 0) {
    fetch_any(ra, b0);
    fetch_any(rb, min(b0 + 1, last));
    stash_any(ra, 0, b0);
    fetch_any(ra, min(b0 + 2, last));
    stash_any(rb, 1, min(b0 + 1, last));
    fetch_any(rb, min(b0 + 3, last));
    stash_any(ra, 2, min(b0 + 2, last));
    fetch_any(ra, min(b0 + 4, last));
    stage_barrier();
    if (live) scores(0, sa_);
  }
  int i = 0;
  for (; i + 1 < nblk; i += 2) {
    step(rb, i, sa_, sb_);      // slot rb holds the odd blocks, ra the even; scores alternate sa_/sb_
    step(ra, i + 1, sb_, sa_);
  }
  if (i < nblk) step(rb, i, sa_, sb_);
  if (!live) return;
  prefill_finish<D, G, NT>(a, st, q0, C, cq0, g, split, qk_scale, vscale, lane, lsum);
}

// Merge of the key splits: one thread per float4 of the output (query row, kv head g,
// head h, 4 dims), combining the nsplit records with log-sum-exp weights; the thread
// at dim 0 writes the row's log-sum-exp.  Records of a split that saw no key of the
// row (lse = -inf) weigh nothing.
constexpr int kPfMergeThreads = 256;

template <int D, int G>
__global__ __launch_bounds__(kPfMergeThreads) void prefill_merge_kernel(AttnArgs a) {
  if (halted(a.cache)) return;
  constexpr int CH = G * D / 4;  // float4 chunks per (row, kv head)
  const int Hkv = a.cache.num_kv_heads, nsplit = a.max_splits;
  const int64_t idx = int64_t(blockIdx.x) * kPfMergeThreads + threadIdx.x;
  if (idx >= int64_t(a.total_q) * Hkv * CH) return;
  const int ch = int(idx % CH);
  const int64_t rg = idx / CH;  // row * Hkv + g
  const int g = int(rg % Hkv);
  const int64_t row = rg / Hkv;
  const int e = ch * 4, h = e / D, d = e % D;
  float m = -INFINITY, w = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // kMergeBatch splits per round, every load of a round issued before any is used
  // (loads past the last split repeat it and are not used): one memory round trip each.
  constexpr int KB = kMergeBatch;
  for (int i0 = 0; i0 < nsplit; i0 += KB) {
    float x[KB];
    float4 o[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int64_t rec = rg * nsplit + min(i0 + u, nsplit - 1);
      x[u] = a.ws_lse[rec * G + h];
      o[u] = *reinterpret_cast<const float4*>(a.ws_o + rec * (G * D) + e);
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (i0 + u >= nsplit) break;
      if (x[u] == -INFINITY) continue;
      const float mn = fmaxf(m, x[u]);
      const float sa = __expf(m - mn), sb = __expf(x[u] - mn);  // m = -inf: sa = 0
      acc.x = acc.x * sa + o[u].x * sb;
      acc.y = acc.y * sa + o[u].y * sb;
      acc.z = acc.z * sa + o[u].z * sb;
      acc.w = acc.w * sa + o[u].w * sb;
      w = w * sa + sb;
      m = mn;
    }
  }
  const float inv = 1.f / w;
  uint16_t* out = static_cast<uint16_t*>(a.out) + (row * a.num_q_heads + g * G + h) * D + d;
  const uint32_t lo = f32_to_bf16(acc.x * inv) | (f32_to_bf16(acc.y * inv) << 16);
  const uint32_t hi = f32_to_bf16(acc.z * inv) | (f32_to_bf16(acc.w * inv) << 16);
  *reinterpret_cast<uint2*>(out) = make_uint2(lo, hi);
  if (a.lse_out && d == 0) a.lse_out[row * a.num_q_heads + g * G + h] = m + __logf(w);
}

template <int KV, int D, int G, bool SMALLP>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  const int groups = a.seqs.num_seqs * a.cache.num_kv_heads * a.max_splits;
  const int64_t grid = int64_t((groups + kXcds - 1) / kXcds) * kXcds * a.pf_qtiles;
  if (SMALLP || a.pf_per_wave) {  // one wave per item (pages of fewer than 32 tokens, short chunks)
    hipLaunchKernelGGL((prefill_kernel<KV, D, G, SMALLP>), dim3(unsigned(grid)), dim3(64), 0, st, a);
  } else {
    hipLaunchKernelGGL((prefill_lds_kernel<KV, D, G>), dim3(unsigned(grid)), dim3(64 * kPfWaves), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  const int64_t threads = int64_t(a.total_q) * a.cache.num_kv_heads * (G * D / 4);
  hipLaunchKernelGGL((prefill_merge_kernel<D, G>), dim3(unsigned((threads + kPfMergeThreads - 1) / kPfMergeThreads)),
                     dim3(kPfMergeThreads), 0, st, a);
  return hipGetLastError();
}

template <int KV, int D, int G>
hipError_t dispatch_p(const AttnArgs& a, hipStream_t st) {
  if constexpr (KV == DT_MXFP4) {
    return a.cache.page_size >= BT ? launch_t<KV, D, G, false>(a, st) : hipErrorInvalidValue;
  } else {
    return a.cache.page_size >= BT ? launch_t<KV, D, G, false>(a, st) : launch_t<KV, D, G, true>(a, st);
  }
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

// Chunks that at most two waves' tiles cover (up to 2 x kPrefillTiles x 16/G queries,
// e.g. 16 tokens verified per sequence at G = 4, D = 128) run on the per-wave kernel: a
// workgroup of the LDS-shared kernel covers kPfTiles x kPfWaves x 16/G queries (64 at
// G = 4), so on such chunks most of its rows would be empty while it still stages every
// block; one or two waves per (sequence, kv head, key split), on one XCD, stream each
// block instead (the second from L2).  Measured on the Llama-shaped batch, 64 sequences:
// 8 tokens 122 us (LDS-shared 284), 16 tokens 158 us (290); from 32 tokens the
// LDS-shared kernel is as fast or faster (32: 296 against 303 us; 64: 307 against 510).
void mfma_prefill_geometry(int kv_dtype, int head_dim, int group, int page_size, int max_q_len,
                           int* queries_per_item, int* resident_items, int* per_wave) {
  const int wave_queries = (16 / group) * (head_dim == 128 ? kPrefillTiles<128> : kPrefillTiles<64>);
  const bool pw = page_size < BT || max_q_len <= 2 * wave_queries;
  *per_wave = pw;
  *queries_per_item = pw ? wave_queries : (16 / group) * kPfTiles * kPfWaves;
  const void* k;
  if (!pw) {
    k = kv_dtype == DT_BF16 ? (head_dim == 64 ? reinterpret_cast<const void*>(&prefill_lds_kernel<DT_BF16, 64, 4>)
                                              : reinterpret_cast<const void*>(&prefill_lds_kernel<DT_BF16, 128, 4>))
        : kv_dtype == DT_FP8 ? (head_dim == 64 ? reinterpret_cast<const void*>(&prefill_lds_kernel<DT_FP8, 64, 4>)
                                               : reinterpret_cast<const void*>(&prefill_lds_kernel<DT_FP8, 128, 4>))
                             : (head_dim == 64 ? reinterpret_cast<const void*>(&prefill_lds_kernel<DT_MXFP4, 64, 4>)
                                               : reinterpret_cast<const void*>(&prefill_lds_kernel<DT_MXFP4, 128, 4>));
  } else if (page_size >= BT) {
    k = kv_dtype == DT_BF16 ? (head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<DT_BF16, 64, 4, false>)
                                              : reinterpret_cast<const void*>(&prefill_kernel<DT_BF16, 128, 4, false>))
        : kv_dtype == DT_FP8 ? (head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<DT_FP8, 64, 4, false>)
                                               : reinterpret_cast<const void*>(&prefill_kernel<DT_FP8, 128, 4, false>))
                             : (head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<DT_MXFP4, 64, 4, false>)
                                               : reinterpret_cast<const void*>(&prefill_kernel<DT_MXFP4, 128, 4, false>));
  } else {
    k = kv_dtype == DT_BF16
            ? (head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<DT_BF16, 64, 4, true>)
                              : reinterpret_cast<const void*>(&prefill_kernel<DT_BF16, 128, 4, true>))
            : (head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<DT_FP8, 64, 4, true>)
                              : reinterpret_cast<const void*>(&prefill_kernel<DT_FP8, 128, 4, true>));
  }
  *resident_items = resident_blocks(k, pw ? 64 : 64 * kPfWaves);
}

hipError_t launch_mfma_prefill(const AttnArgs& a, hipStream_t st) {
  if (a.seqs.num_seqs == 0 || a.total_q == 0) return hipSuccess;
  switch (a.cache.dtype) {
    case DT_BF16: return dispatch_d<DT_BF16>(a, st);
    case DT_FP8: return dispatch_d<DT_FP8>(a, st);
    case DT_MXFP4: return dispatch_d<DT_MXFP4>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
