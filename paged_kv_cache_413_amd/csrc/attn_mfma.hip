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
//   K tile of a page is token-major [P][D]: lane (m, c) loads 8 dims of one token row;
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
// sequences); a range that covers a whole (sequence, kv head) writes the output
// directly, a cut one writes a normalised partial and its log-sum-exp, and a small
// merge kernel combines the pieces exactly (log-sum-exp weights).  "fixed" gives each
// page-aligned partition of a fixed size its own wave, as in a conventional split-KV
// decode, with the same merge.  (Merging inside the decode kernel, by the last wave
// to finish a piece, needs agent-scope release/acquire fences; on this chip those
// write back and invalidate a whole L2 per piece, which costs far more than the
// second launch.)
#include "device_common.h"
#include "internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int BT = 32;      // tokens per block
constexpr int LOG2_BT = 5;

// Cache-policy bits of the K/V buffer loads (0 = default; the data is read once).
#ifndef PKV_KV_LOAD_AUX
#define PKV_KV_LOAD_AUX 0
#endif
// Waves per SIMD the decode kernels are compiled for (register budget 512 / this).
#ifndef PKV_DECODE_WAVES_PER_EU
#define PKV_DECODE_WAVES_PER_EU 2
#endif
// Blocks whose loads are in flight while one is folded, plus one (2 or 3 buffers).
#ifndef PKV_DECODE_DEPTH
#define PKV_DECODE_DEPTH 2
#endif

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

union Frag8 {
  bf16x8 v;
  uint32_t w[4];
  uint4 q;
};

// Eight consecutive cache elements at byte offset `off` of the wave-uniform address
// `base`, as bf16.  bf16: a 16-byte load.  FP8 E4M3: an 8-byte load, each code widened
// exactly (every E4M3 value is a bf16 value).
template <int KV>
__device__ __forceinline__ bf16x8 load8(const char* __restrict__ base, uint32_t off) {
  Frag8 f;
  if constexpr (KV == DT_BF16) {
    f.q = *reinterpret_cast<const uint4*>(base + off);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(base + off);
    f.w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false));
    f.w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true));
    f.w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false));
    f.w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true));
  }
  return f.v;
}

// Buffer descriptor of one tile (wave-uniform, 4 scalar registers): loads address it
// with the lane's fixed 32-bit offset plus a scalar offset, and anything past the
// tile's `bytes` reads as zero instead of touching other memory.  Word 3 is the
// gfx9-family default (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, int(bytes), 0x00020000);
}

template <int KV>
__device__ __forceinline__ bf16x8 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  Frag8 f;
  if constexpr (KV == DT_BF16) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, PKV_KV_LOAD_AUX));
    f.w[0] = v[0];
    f.w[1] = v[1];
    f.w[2] = v[2];
    f.w[3] = v[3];
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, PKV_KV_LOAD_AUX));
    f.w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false));
    f.w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true));
    f.w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false));
    f.w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true));
  }
  return f.v;
}

// Four consecutive cache elements at byte offset `off`, as bf16 in words 0 and 1.
template <int KV>
__device__ __forceinline__ Frag8 load4x2(const char* __restrict__ base, uint32_t off) {
  Frag8 f;
  f.q = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (KV == DT_BF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(base + off);
    f.w[0] = w.x;
    f.w[1] = w.y;
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(base + off);
    f.w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    f.w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  }
  return f;
}

__device__ __forceinline__ bf16x8 zero8() {
  Frag8 f;
  f.q = make_uint4(0u, 0u, 0u, 0u);
  return f.v;
}

template <int D>
struct Block {
  bf16x8 ka[D / 32], kb[D / 32];  // K of tokens 0..15 and 16..31, D/32 dim chunks each
  bf16x8 v[D / 16];               // V: D/16 tiles of 16 dims x 32 tokens
};

// Token (0..31 within the block) behind element e of lane group c of the P and V
// operands.
__device__ __forceinline__ int tok_of(int c, int e) { return e < 4 ? 4 * c + e : 12 + 4 * c + e; }

// Per-lane byte offsets, fixed for the whole range: lane (m, c) reads K row m of the
// block (sub-tile a; +16 rows for b) at dims 8c.. of a 32-dim chunk, and V dim m
// (+16 per V tile) at positions 8c.. of the block's 32-slot V sub-block.
struct LaneOffsets {
  uint32_t k, v;
};

template <int KV, int D>
__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
  constexpr int esz = KV == DT_BF16 ? 2 : 1;
  const int m = lane & 15, c = lane >> 4;
  return {uint32_t((m * 32 + 8 * c) * esz), uint32_t((m * BT + 8 * c) * esz)};
}

// 64 consecutive block-table entries of one sequence, one per lane: the page of a
// block is read from a register (readlane), so no table load sits between one
// block's loads and the next.  `base` is the logical page of lane 0.
struct PageWindow {
  int32_t ids;
  int base;
};

// Load the window starting at logical page `base` of a table row with `npages`
// valid entries (entries past them read as 0 and are never used).
__device__ __forceinline__ void load_window(PageWindow& w, const int32_t* __restrict__ bt, int base,
                                            int npages, int lane) {
  w.base = base;
  w.ids = base + lane < npages ? bt[base + lane] : 0;
}

// Page of logical page p, refilling the window when p has left it (at most once per
// 64 pages).
__device__ __forceinline__ int32_t page_of(PageWindow& w, const int32_t* __restrict__ bt, int p,
                                           int npages, int lane) {
  if (p - w.base >= 64) load_window(w, bt, p, npages, lane);
  return __builtin_amdgcn_readlane(w.ids, p - w.base);
}

// Issue the loads of the block starting at token t (a multiple of 32) of the sequence
// whose table row is bt.  With pages of >= 32 tokens the block lies in one page, whose
// id comes from the page window, and every address is that page's tile base
// (uniform) plus the lane's fixed offset.  Shorter pages (SMALLP) take the page of
// each lane's own tokens from the table, and skip tokens at or past L (the sequence
// length): their page may not exist.
template <int KV, int D, bool SMALLP>
__device__ __forceinline__ void load_block(Block<D>& b, const char* __restrict__ pool,
                                           const int32_t* __restrict__ bt, PageWindow& win, int t,
                                           int L, int log2P, int64_t kv_stride_b, int64_t head_off_b,
                                           LaneOffsets lo, int lane) {
  constexpr int esz = KV == DT_BF16 ? 2 : 1;
  const int P = 1 << log2P;
  if constexpr (!SMALLP) {
    const int32_t page = page_of(win, bt, t >> log2P, (L + P - 1) >> log2P, lane);
    const uint32_t slot0 = uint32_t(t & (P - 1));
    const uint32_t tile_bytes = uint32_t(P) * D * esz;
    const char* K = pool + int64_t(page) * 2 * kv_stride_b + head_off_b;
    const auto rk = tile_rsrc(K, tile_bytes);
    const auto rv = tile_rsrc(K + kv_stride_b, tile_bytes);
    const uint32_t ks = slot0 * 32 * esz, vs = slot0 * D * esz;  // V: sub-block slot0/32
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {  // chunk j: 16 rows x 64 B, one contiguous run each
      const uint32_t kj = __builtin_amdgcn_readfirstlane(ks + uint32_t(j * 32 * esz) * P);
      b.ka[j] = bload8<KV>(rk, lo.k, kj);
      b.kb[j] = bload8<KV>(rk, lo.k + 16 * 32 * esz, kj);
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)  // 16 dims x 32 tokens: one contiguous run
      b.v[dt] = bload8<KV>(rv, lo.v, __builtin_amdgcn_readfirstlane(vs + uint32_t(16 * BT * dt * esz)));
  } else {
    // pages of 8 or 16 slots: V tiles are [D][P] in natural slot order
    const int m = lane & 15, c = lane >> 4;
    const int P1 = P - 1;
    const int ta = t + m, tb = ta + 16;
    const uint32_t kcol = uint32_t(8 * c * esz);
    if (ta < L) {
      const char* K = pool + int64_t(bt[ta >> log2P]) * 2 * kv_stride_b + head_off_b;
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
        b.ka[j] = load8<KV>(K, uint32_t(((j << log2P) + (ta & P1)) * 32 * esz) + kcol);
    } else {
#pragma unroll
      for (int j = 0; j < D / 32; ++j) b.ka[j] = zero8();
    }
    if (tb < L) {
      const char* K = pool + int64_t(bt[tb >> log2P]) * 2 * kv_stride_b + head_off_b;
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
        b.kb[j] = load8<KV>(K, uint32_t(((j << log2P) + (tb & P1)) * 32 * esz) + kcol);
    } else {
#pragma unroll
      for (int j = 0; j < D / 32; ++j) b.kb[j] = zero8();
    }
    // V: tokens 4c..4c+3 (elements 0..3) and 16+4c..16+4c+3 (elements 4..7), four
    // consecutive slots of one page each
    const int t0 = t + 4 * c, t1 = t0 + 16;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      Frag8 f;
      f.q = make_uint4(0u, 0u, 0u, 0u);
      if (t0 < L) {
        const char* V = pool + (int64_t(bt[t0 >> log2P]) * 2 + 1) * kv_stride_b + head_off_b;
        const Frag8 h = load4x2<KV>(V, uint32_t((((16 * dt + m) << log2P) + (t0 & P1)) * esz));
        f.w[0] = h.w[0];
        f.w[1] = h.w[1];
      }
      if (t1 < L) {
        const char* V = pool + (int64_t(bt[t1 >> log2P]) * 2 + 1) * kv_stride_b + head_off_b;
        const Frag8 h = load4x2<KV>(V, uint32_t((((16 * dt + m) << log2P) + (t1 & P1)) * esz));
        f.w[2] = h.w[0];
        f.w[3] = h.w[1];
      }
      b.v[dt] = f.v;
    }
  }
}

// Online-softmax state of one wave: running max m (log2 units, per head lane), the
// lane's share of the running sum, and the output accumulator O [16 heads x D]
// (lane (n, c) holds heads 4c..4c+3 of dim 16*dt + n in O[dt]).
template <int D>
struct State {
  float m, l;
  f32x4 o[D / 16];
};

template <int D>
__device__ __forceinline__ void state_init(State<D>& st) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Fold one block into the state.  t_end: first token past this range; when the
// block reaches past it (the range's last block) the scores of the excess tokens are
// masked and their V entries zeroed (their slots may hold anything, NaN included).
template <int D>
__device__ __forceinline__ void fold_block(State<D>& st, Block<D>& b, const bf16x8 (&qf)[D / 32],
                                           float qk_scale, int t, int t_end, int lane) {
  const int c = lane >> 4;
  f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    sa = mma(b.ka[j], qf[j], sa);
    sb = mma(b.kb[j], qf[j], sb);
  }
  float sc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = sa[i] * qk_scale;
    sc[4 + i] = sb[i] * qk_scale;
  }
  if (t + BT > t_end) {  // wave-uniform: the range's last, partial block
    const int nvalid = t_end - t;  // tokens of the block still in range
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (tok_of(c, e) >= nvalid) sc[e] = -INFINITY;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      Frag8 f;
      f.v = b.v[dt];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t keep = (tok_of(c, 2 * w) < nvalid ? 0x0000ffffu : 0u) |
                              (tok_of(c, 2 * w + 1) < nvalid ? 0xffff0000u : 0u);
        f.w[w] &= keep;
      }
      b.v[dt] = f.v;
    }
  }
  float bm = sc[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sc[e]);
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  const float mn = fmaxf(st.m, bm);
  const float alpha = exp2f(st.m - mn);  // 0 on the first block (m = -inf)
  float p[8], ps = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = exp2f(sc[e] - mn);
    ps += p[e];
  }
  st.l = st.l * alpha + ps;
  if (__ballot(mn != st.m)) {  // some head's max moved: rescale O by that head's alpha
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * c + i, 64);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.o[dt][i] *= al[i];
  }
  st.m = mn;
  Frag8 pa;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    pa.w[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2 * w], p[2 * w + 1]}, bf16x2));
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.o[dt] = mma(pa.v, b.v[dt], st.o[dt]);
}

// Blocks [b0, b1) of one (sequence, kv head), t_end = last token + 1 of the range.
// PKV_DECODE_DEPTH register buffers rotate: while block i is folded the loads of the
// next DEPTH-1 blocks are in flight.  Inside the loop every prefetch is
// unconditional, so each fold waits only for its own block's loads (a partial
// vmcnt), never for prefetches issued after them; the last blocks are peeled.
template <int KV, int D, bool SMALLP>
__device__ __forceinline__ void run_range(State<D>& st, const bf16x8 (&qf)[D / 32], float qk_scale,
                                          const char* __restrict__ pool, const int32_t* __restrict__ bt,
                                          int b0, int b1, int t_end, int L, int log2P,
                                          int64_t kv_stride_b, int64_t head_off_b, int lane) {
  const LaneOffsets lo = lane_offsets<KV, D>(lane);
  PageWindow win;
  if constexpr (!SMALLP) load_window(win, bt, (b0 << LOG2_BT) >> log2P, (L + (1 << log2P) - 1) >> log2P, lane);
  auto ld = [&](Block<D>& b, int blk) {
    load_block<KV, D, SMALLP>(b, pool, bt, win, blk << LOG2_BT, L, log2P, kv_stride_b, head_off_b, lo, lane);
  };
  auto fold = [&](Block<D>& b, int blk) { fold_block<D>(st, b, qf, qk_scale, blk << LOG2_BT, t_end, lane); };
  Block<D> x, y;
  ld(x, b0);
  int blk = b0;
  if constexpr (PKV_DECODE_DEPTH == 2) {
    for (; blk + 2 < b1; blk += 2) {
      ld(y, blk + 1);
      fold(x, blk);
      ld(x, blk + 2);
      fold(y, blk + 1);
    }
    if (blk + 1 < b1) {
      ld(y, blk + 1);
      fold(x, blk);
      fold(y, blk + 1);
    } else {
      fold(x, blk);
    }
  } else {
    Block<D> z;
    if (b1 - b0 == 1) {
      fold(x, blk);
      return;
    }
    ld(y, b0 + 1);
    for (; blk + 4 < b1; blk += 3) {
      ld(z, blk + 2);
      fold(x, blk);
      ld(x, blk + 3);
      fold(y, blk + 1);
      ld(y, blk + 4);
      fold(z, blk + 2);
    }
    const int r = b1 - blk;  // 2..4 blocks left; x and y hold blk, blk+1
    if (r == 2) {
      fold(x, blk);
      fold(y, blk + 1);
    } else if (r == 3) {
      ld(z, blk + 2);
      fold(x, blk);
      fold(y, blk + 1);
      fold(z, blk + 2);
    } else {
      ld(z, blk + 2);
      fold(x, blk);
      ld(x, blk + 3);
      fold(y, blk + 1);
      fold(z, blk + 2);
      fold(x, blk + 3);
    }
  }
}

// Q^T operand of query row `row`, kv head g: lane (n, c) holds dims 32j + 8c .. +7 of
// query head g*G + n (zero for n >= G).  Queries are bf16.
template <int D, int G>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[D / 32], const void* __restrict__ q, int row,
                                       int Hq, int g, int lane) {
  const int n = lane & 15, c = lane >> 4;
  if (n < G) {
    const uint16_t* base = static_cast<const uint16_t*>(q) + (int64_t(row) * Hq + g * G + n) * D + 8 * c;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      Frag8 f;
      f.q = *reinterpret_cast<const uint4*>(base + 32 * j);
      qf[j] = f.v;
    }
  } else {
#pragma unroll
    for (int j = 0; j < D / 32; ++j) qf[j] = zero8();
  }
}

// Merge the n partial records of one (query row, kv head) -- record i is rec(i) --
// into the final output and log-sum-exp: LSE_h = log sum_i exp(lse_ih),
// out_h = sum_i exp(lse_ih - LSE_h) o_ih.  One 256-thread workgroup: every thread
// owns float4 chunks of the G x D record (one head each) and a stride of records,
// and keeps a running (max, sum of weights, weighted sum) over them, so the loads
// of different records are independent and in flight together; the record-parallel
// states are then combined in LDS.
constexpr int kMergeThreads = 256;

template <int D, int G, typename RecFn>
__device__ __forceinline__ void merge_partials(const AttnArgs& a, int row, int g, int n, RecFn rec) {
  constexpr int NT = kMergeThreads;
  constexpr int C = G * D / 4;                  // float4 chunks per record
  constexpr int CC = C < NT ? C : NT;           // chunk lanes
  constexpr int RP = NT / CC;                   // record-parallel factor
  constexpr int CPT = (C + NT - 1) / NT;        // chunks per thread
  __shared__ float4 s_acc[RP][CC * CPT];
  __shared__ float s_m[RP][CC * CPT], s_w[RP][CC * CPT];
  const int t = threadIdx.x;
  const int cl = t % CC, rp = t / CC;
  float4 acc[CPT];
  float m[CPT], w[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    m[k] = -INFINITY;
    w[k] = 0.f;
  }
#pragma unroll 4
  for (int i = rp; i < n; i += RP) {
    const int64_t r = rec(i);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int e = (cl + k * CC) * 4;
      if (e < G * D) {
        const float x = a.ws_lse[r * G + e / D];
        const float4 o = *reinterpret_cast<const float4*>(a.ws_o + r * (G * D) + e);
        const float mn = fmaxf(m[k], x);
        const float sa = __expf(m[k] - mn), sb = __expf(x - mn);  // m = -inf: sa = 0
        acc[k].x = acc[k].x * sa + o.x * sb;
        acc[k].y = acc[k].y * sa + o.y * sb;
        acc[k].z = acc[k].z * sa + o.z * sb;
        acc[k].w = acc[k].w * sa + o.w * sb;
        w[k] = w[k] * sa + sb;
        m[k] = mn;
      }
    }
  }
  if constexpr (RP > 1) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      s_acc[rp][cl + k * CC] = acc[k];
      s_m[rp][cl + k * CC] = m[k];
      s_w[rp][cl + k * CC] = w[k];
    }
    __syncthreads();
    if (rp != 0) return;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      for (int q = 1; q < RP; ++q) {
        const float mo = s_m[q][cl + k * CC];
        if (mo == -INFINITY) continue;  // that lane had no records
        const float4 o = s_acc[q][cl + k * CC];
        const float mn = fmaxf(m[k], mo);
        const float sa = __expf(m[k] - mn), sb = __expf(mo - mn);
        acc[k].x = acc[k].x * sa + o.x * sb;
        acc[k].y = acc[k].y * sa + o.y * sb;
        acc[k].z = acc[k].z * sa + o.z * sb;
        acc[k].w = acc[k].w * sa + o.w * sb;
        w[k] = w[k] * sa + s_w[q][cl + k * CC] * sb;
        m[k] = mn;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int e = (cl + k * CC) * 4;
    if (e < G * D) {
      const int h = e / D, d = e % D;
      const float inv = 1.f / w[k];
      uint16_t* o = static_cast<uint16_t*>(a.out) + (int64_t(row) * a.num_q_heads + g * G + h) * D + d;
      const uint32_t lo = f32_to_bf16(acc[k].x * inv) | (f32_to_bf16(acc[k].y * inv) << 16);
      const uint32_t hi = f32_to_bf16(acc[k].z * inv) | (f32_to_bf16(acc[k].w * inv) << 16);
      *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
      if (a.lse_out && d == 0) a.lse_out[int64_t(row) * a.num_q_heads + g * G + h] = m[k] + __logf(w[k]);
    }
  }
}

// Finish a range: reduce the running sum over the four lane groups of each head and
// normalise.  A range that covers its whole (query row, kv head) writes the output
// (bf16) and log-sum-exp directly; a cut one writes partial record `rec`:
// ws_o[rec][G][D] (normalised) and ws_lse[rec][G], merged by the merge kernel.
template <int D, int G>
__device__ __forceinline__ void finish(const State<D>& st, const AttnArgs& a, int row, int g,
                                       bool complete, int64_t rec, float vscale, int lane) {
  const int nn = lane & 15, c = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const float lse = (st.m + __log2f(l)) * kLn2;  // natural log, valid in lanes nn < G
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) inv[i] = vscale / __shfl(l, 4 * c + i, 64);
  const int Hq = a.num_q_heads;
  if (complete) {
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * c + i;
      if (h < G) {
        uint16_t* o = out + (int64_t(row) * Hq + g * G + h) * D + nn;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[16 * dt] = uint16_t(f32_to_bf16(st.o[dt][i] * inv[i]));
      }
    }
    if (a.lse_out && c == 0 && nn < G) a.lse_out[int64_t(row) * Hq + g * G + nn] = lse;
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * c + i;
    if (h < G) {
      float* o = a.ws_o + (rec * G + h) * D + nn;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[16 * dt] = st.o[dt][i] * inv[i];
    }
  }
  if (c == 0 && nn < G) a.ws_lse[rec * G + nn] = lse;
}

template <int KV>
__device__ __forceinline__ void scales(const AttnArgs& a, int g, float& qk_scale, float& vscale) {
  qk_scale = a.sm_scale * kLog2e;
  vscale = 1.f;
  if constexpr (KV == DT_FP8) {
    qk_scale *= a.cache.k_scale[g];
    vscale = a.cache.v_scale[g];
  }
}

// ---- fixed partitions: one wave per (sequence, kv head, partition) ---------------------
template <int KV, int D, int G, bool SMALLP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(PKV_DECODE_WAVES_PER_EU, PKV_DECODE_WAVES_PER_EU))) void decode_fixed_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  const int split = blockIdx.x % a.max_splits;
  const int sg = blockIdx.x / a.max_splits;
  const int Hkv = a.cache.num_kv_heads;
  const int g = sg % Hkv, s = sg / Hkv;
  const int L = a.seqs.context_lens[s];
  const int t0 = split * a.chunk;
  if (t0 >= L) return;
  const int t1 = min(L, t0 + a.chunk);
  const int nsplit = (L + a.chunk - 1) / a.chunk;
  float qk_scale, vscale;
  scales<KV>(a, g, qk_scale, vscale);
  bf16x8 qf[D / 32];
  load_q<D, G>(qf, a.q, s, a.num_q_heads, g, lane);
  State<D> st;
  state_init(st);
  constexpr int esz = KV == DT_BF16 ? 2 : 1;
  const int64_t tile_b = int64_t(a.cache.page_size) * D * esz;
  const int32_t* bt = a.seqs.block_tables + int64_t(s) * a.seqs.max_pages_per_seq;
  run_range<KV, D, SMALLP>(st, qf, qk_scale, static_cast<const char*>(a.cache.pool), bt,
                           t0 >> LOG2_BT, (t1 + BT - 1) >> LOG2_BT, t1, L, a.cache.log2_page,
                           Hkv * tile_b, g * tile_b, lane);
  finish<D, G>(st, a, s, g, nsplit == 1, int64_t(sg) * a.max_splits + split, vscale, lane);
}

// ---- auto: contiguous equal shares of the flattened block space ------------------------
// Flattened order: sequence-major, then kv head, then block; segment (s, g) covers
// [Hkv*cum_s + g*nb_s, +nb_s) with nb_s = ceil(L_s / 32) and cum_s = sum_{s'<s} nb_s'.

// A value every lane holds equally, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// Total blocks of all (sequence, kv head) segments.
__device__ __forceinline__ int64_t total_blocks(const int32_t* __restrict__ lens, int S, int Hkv,
                                                int lane) {
  int64_t sum = 0;
  for (int s = lane; s < S; s += 64) sum += (lens[s] + BT - 1) >> LOG2_BT;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  return uniform64(sum * Hkv);
}

// Sequence whose segments contain flat block f, and its cum (blocks before it).
__device__ __forceinline__ void locate(const int32_t* __restrict__ lens, int S, int Hkv, int64_t f,
                                       int lane, int& s_out, int64_t& cum_out) {
  int64_t run = 0;
  for (int base = 0; base < S; base += 64) {
    const int s = base + lane;
    const int64_t nb = s < S ? int64_t((lens[s] + BT - 1) >> LOG2_BT) : 0;
    const int64_t incl = wave_incl_scan(nb, lane);
    const uint64_t hit = __ballot(s < S && Hkv * (run + incl) > f);
    if (hit) {
      const int first = __builtin_ctzll(hit);
      s_out = base + first;
      cum_out = uniform64(run + __shfl(incl - nb, first, 64));
      return;
    }
    run = uniform64(run + __shfl(incl, 63, 64));
  }
  s_out = S;
  cum_out = run;
}

template <int KV, int D, int G, bool SMALLP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(PKV_DECODE_WAVES_PER_EU, PKV_DECODE_WAVES_PER_EU))) void decode_auto_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  const int w = blockIdx.x;
  const int S = a.seqs.num_seqs, Hkv = a.cache.num_kv_heads;
  const int32_t* lens = a.seqs.context_lens;
  const int64_t T = total_blocks(lens, S, Hkv, lane);
  const int64_t share = max(int64_t(a.min_share), (T + a.num_waves - 1) / a.num_waves);
  const int64_t f0 = int64_t(w) * share;
  int4* desc = a.ws_desc + w;
  if (f0 >= T) {
    if (lane == 0) *desc = make_int4(-1, 0, 0, 0);
    return;
  }
  const int64_t fend = min(T, f0 + share);
  int s;
  int64_t cum;
  locate(lens, S, Hkv, f0, lane, s, cum);
  constexpr int esz = KV == DT_BF16 ? 2 : 1;
  const int64_t tile_b = int64_t(a.cache.page_size) * D * esz;
  int64_t f = f0;
  bool first = true;
  while (f < fend) {
    const int L = lens[s];
    const int nb = (L + BT - 1) >> LOG2_BT;
    const int64_t seg0 = Hkv * cum;
    const int g = int((f - seg0) / nb);
    const int64_t gs = seg0 + int64_t(g) * nb;            // this segment's first flat block
    const int b0 = int(f - gs);
    const int b1 = int(min(int64_t(nb), fend - gs));
    if (first && lane == 0) {
      // This wave merges its first segment when that segment started in an earlier
      // wave (w0) and ends inside this one.  Record slot of w0: 1 unless the segment
      // is w0's first too.
      const int64_t w0 = gs / share;
      const bool merges = gs < f0 && gs + nb <= fend;
      *desc = make_int4(s, g, int(w0), merges ? (1 | (gs != w0 * share ? 2 : 0)) : 0);
    }
    float qk_scale, vscale;
    scales<KV>(a, g, qk_scale, vscale);
    bf16x8 qf[D / 32];
    load_q<D, G>(qf, a.q, s, a.num_q_heads, g, lane);
    State<D> st;
    state_init(st);
    const int32_t* bt = a.seqs.block_tables + int64_t(s) * a.seqs.max_pages_per_seq;
    const int t_end = min(L, b1 << LOG2_BT);
    run_range<KV, D, SMALLP>(st, qf, qk_scale, static_cast<const char*>(a.cache.pool), bt, b0, b1,
                             t_end, L, a.cache.log2_page, Hkv * tile_b, g * tile_b, lane);
    const bool complete = b0 == 0 && b1 == nb;
    finish<D, G>(st, a, s, g, complete, int64_t(w) * 2 + (first ? 0 : 1), vscale, lane);
    first = false;
    f = gs + b1;
    if (g + 1 == Hkv) {
      cum += nb;
      ++s;
    }
  }
}

// Merge of one cut (sequence, kv head) segment of the balanced schedule, by the
// workgroup of the wave that holds its last piece (a wave is the last one of at
// most one cut segment: its first).  The pieces are in waves w0 .. w; the record of
// wave v is slot 0, except slot 1 for w0 when the segment is not w0's first.
template <int D, int G>
__global__ __launch_bounds__(kMergeThreads) void merge_auto_kernel(AttnArgs a) {
  const int w = blockIdx.x;
  const int4 d = a.ws_desc[w];  // (sequence, kv head, w0, flags)
  if (d.x < 0 || !(d.w & 1)) return;
  const int64_t w0 = d.z;
  const bool slot1 = d.w & 2;
  merge_partials<D, G>(a, d.x, d.y, int(w - w0 + 1),
                       [w0, slot1](int i) { return (w0 + i) * 2 + ((i == 0 && slot1) ? 1 : 0); });
}

// Merge of the fixed partitions of one (sequence, kv head).
template <int D, int G>
__global__ __launch_bounds__(kMergeThreads) void merge_fixed_kernel(AttnArgs a) {
  const int sg = blockIdx.x;
  const int Hkv = a.cache.num_kv_heads;
  const int g = sg % Hkv, s = sg / Hkv;
  const int n = (a.seqs.context_lens[s] + a.chunk - 1) / a.chunk;
  if (n <= 1) return;  // written directly
  const int64_t r0 = int64_t(sg) * a.max_splits;
  merge_partials<D, G>(a, s, g, n, [r0](int i) { return r0 + i; });
}

// ---- host side ---------------------------------------------------------------------------

template <int KV, int D, int G, bool SMALLP>
hipError_t launch_t(const AttnArgs& a, const MfmaPlan& p, hipStream_t st) {
  if (p.auto_mode) {
    hipLaunchKernelGGL((decode_auto_kernel<KV, D, G, SMALLP>), dim3(p.waves), dim3(64), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((merge_auto_kernel<D, G>), dim3(p.waves), dim3(kMergeThreads), 0, st, a);
    return hipGetLastError();
  }
  const int64_t nblk = int64_t(a.seqs.num_seqs) * a.cache.num_kv_heads * a.max_splits;
  hipLaunchKernelGGL((decode_fixed_kernel<KV, D, G, SMALLP>), dim3(unsigned(nblk)), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL((merge_fixed_kernel<D, G>), dim3(unsigned(int64_t(a.seqs.num_seqs) * a.cache.num_kv_heads)),
                     dim3(kMergeThreads), 0, st, a);
  return hipGetLastError();
}

template <int KV, int D, int G>
hipError_t dispatch_p(const AttnArgs& a, const MfmaPlan& p, hipStream_t st) {
  return a.cache.page_size >= BT ? launch_t<KV, D, G, false>(a, p, st) : launch_t<KV, D, G, true>(a, p, st);
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
const void* auto_kernel_for(int G, bool smallp) {
#define PKV_K(GG) (smallp ? reinterpret_cast<const void*>(&decode_auto_kernel<KV, D, GG, true>) \
                          : reinterpret_cast<const void*>(&decode_auto_kernel<KV, D, GG, false>))
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
  return (kv_dtype == DT_BF16 || kv_dtype == DT_FP8) && q_dtype == DT_BF16 &&
         (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16) && page_size >= 8;
}

int mfma_auto_waves(int kv_dtype, int head_dim, int group, int page_size) {
  const bool smallp = page_size < BT;
  const void* k = kv_dtype == DT_BF16
                      ? (head_dim == 64 ? auto_kernel_for<DT_BF16, 64>(group, smallp)
                                        : auto_kernel_for<DT_BF16, 128>(group, smallp))
                      : (head_dim == 64 ? auto_kernel_for<DT_FP8, 64>(group, smallp)
                                        : auto_kernel_for<DT_FP8, 128>(group, smallp));
  return resident_blocks(k, 64);
}

hipError_t launch_mfma_decode(const AttnArgs& a, const MfmaPlan& p, hipStream_t st) {
  if (a.seqs.num_seqs == 0) return hipSuccess;
  return a.cache.dtype == DT_BF16 ? dispatch_d<DT_BF16>(a, p, st) : dispatch_d<DT_FP8>(a, p, st);
}

}  // namespace pkv
