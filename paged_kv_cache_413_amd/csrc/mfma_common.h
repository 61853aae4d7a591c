// Device building blocks shared by the matrix-core attention kernels (decode and
// prefill): operand types, loads of one 32-token block of a (page, kv head) straight
// into MFMA operand registers, the page-table window, the online-softmax state and
// its per-block update, the block pipeline, and the log-sum-exp merge of partial
// results.  Everything here is wave-level; see attn_mfma.hip for the decode kernels
// and prefill_mfma.hip for the prefill kernels.
//
// Block products (one wave, 16 query rows in the MFMA N dimension):
//   scores^T [32 tok x 16 rows] = K [32 x D] . Q^T [D x 16]   -> 2 x D/32 MFMAs
//   O        [16 rows x D]     += P [16 x 32 tok] . V [32 x D] -> D/16 MFMAs
// with v_mfma_f32_16x16x32_bf16 (fp32 accumulate).  The two K sub-tiles are tokens
// 0..15 and 16..31 of the block, so the scores of row n land in lane (n, c) for tokens
// 4c..4c+3 and 16+4c..16+4c+3 -- the P operand of the second product (k index 8c + e)
// -- and the V sub-block of the pool stores its slots in that same order.
#pragma once

#include <type_traits>

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
constexpr int kXcds = 8;    // MI355X: 8 XCDs, each with its own L2; workgroup b runs on XCD b mod 8

// Cache-policy bits of the decode kernels' K/V buffer loads: 2 = non-temporal (the
// data streams through once per call).  Measured against the default policy: 9-13 %
// faster on batches whose K/V is read once (592 MB Llama batch, 4.3 GB 131k context,
// 5 % on FP8 without shared pages), 3-4 % slower where pages are re-read -- by the 32
// sequences sharing a prefix in one call, or from the 256 MB Infinity Cache across
// calls when the working set nearly fits in it.  The LDS-shared prefill kernel loads with
// the default policy: every query tile of a sequence re-reads its K/V through L2.
#ifndef PKV_KV_LOAD_AUX
#define PKV_KV_LOAD_AUX 2
#endif
// Waves per SIMD the decode kernels are compiled for (register budget 512 / this).
// One: two waves on a SIMD split its share of the bandwidth unevenly (the older one
// issues first and runs about twice as fast while both are active), and with 1024
// single waves the two HBM-bound loads measure 5 % faster than with 2048.
#ifndef PKV_DECODE_WAVES_PER_EU
#define PKV_DECODE_WAVES_PER_EU 1
#endif
// Register buffers of the block pipeline (blocks in flight while one is folded, plus
// one).  MXFP4 blocks (4.25 KiB per wave) are bound by their decoding, not by bytes in
// flight: measured on the Llama batch, two buffers with two waves per SIMD take 41 us
// per call; three or four buffers with two waves 42-43 us; one wave per SIMD 48-53 us
// at any depth; three or four waves per SIMD spill registers (55-100 us).
#ifndef PKV_DECODE_DEPTH
#define PKV_DECODE_DEPTH 2
#endif
#ifndef PKV_MX_DEPTH
#define PKV_MX_DEPTH 2
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

// A value every lane holds equally, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// A 32-bit value every lane holds equally (a load from a wave-uniform address), in a
// scalar register: what is derived from it -- block ranges, loop bounds, tile
// addresses -- stays scalar, and the block loops branch on scalar conditions.
__device__ __forceinline__ int uniform32(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A tile address every lane holds equally, in scalar registers: a buffer descriptor
// built from it is then known to be uniform, and its loads need no per-load check.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  return reinterpret_cast<const char*>(uniform64(reinterpret_cast<int64_t>(p)));
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

// Load the window starting at logical page `base` (< npages) of a table row with
// `npages` valid entries.  Lanes past them repeat the last entry and are never used:
// the load is unconditional, so nothing waits for it before its first use (a masked
// load merged with a constant would make the wave wait right after issuing it).
__device__ __forceinline__ void load_window(PageWindow& w, const int32_t* __restrict__ bt, int base,
                                            int npages, int lane) {
  w.base = base;
  w.ids = bt[min(base + lane, npages - 1)];
}

// Page of logical page p, which lies in the window.
__device__ __forceinline__ int32_t page_of(const PageWindow& w, int p) {
  return __builtin_amdgcn_readlane(w.ids, p - w.base);
}

// Issue the loads of the block starting at token t (a multiple of 32) of the sequence
// whose table row is bt.  With pages of >= 32 tokens the block lies in one page, whose
// id comes from the page window (which must hold it), and every address is that
// page's tile base (uniform) plus the lane's fixed offset.  Shorter pages (SMALLP) take the page of
// each lane's own tokens from the table, and skip tokens at or past L (the sequence
// length): their page may not exist.
template <int KV, int D, bool SMALLP>
__device__ __forceinline__ void load_block(Block<D>& b, const char* __restrict__ pool,
                                           const int32_t* __restrict__ bt, const PageWindow& win, int t,
                                           int L, int log2P, int64_t kv_stride_b, int64_t head_off_b,
                                           LaneOffsets lo, int lane) {
  constexpr int esz = KV == DT_BF16 ? 2 : 1;
  const int P = 1 << log2P;
  if constexpr (!SMALLP) {
    const int32_t page = page_of(win, t >> log2P);
    const uint32_t slot0 = uint32_t(t & (P - 1));
    const uint32_t tile_bytes = uint32_t(P) * D * esz;
    const char* K = uniform_ptr(pool + int64_t(page) * 2 * kv_stride_b + head_off_b);
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

// ---- MXFP4 blocks -------------------------------------------------------------------------
// One 32-token block of an MXFP4 tile in the lane layout of the two products (pages of
// >= 32 tokens), as loaded: E2M1 codes, eight per word, and E8M0 scale bytes.  Lane
// (m, c) holds K dims 32j + 8c .. +7 of tokens m and 16 + m (word j of ka, kb) with
// their scales (byte j of ksa, ksb), the V codes of dims 16u + m at positions 8c .. 8c+7
// (word u of v), and the V scales of those eight positions (position e, block j: byte
// e*(D/32) + j of vs).
template <int D>
struct MxBlock {
  uint32_t ka[D / 32], kb[D / 32];
  uint32_t ksa, ksb;
  uint32_t v[D / 16];
  uint32_t vs[D / 16];
};

// ---- raw FP8 blocks ------------------------------------------------------------------------
// One 32-token block of an FP8 tile (pages of >= 32 tokens) as loaded: the E4M3 codes of
// the lane's operands (8 per uint2, in the lane layout of Block), widened to bf16 only
// when the block is folded (ready).  Half the registers of a widened block: the dense
// decode kernel runs two waves per SIMD with these.
template <int D>
struct F8Block {
  uint2 ka[D / 32], kb[D / 32];
  uint2 v[D / 16];
};

// RAW: FP8 blocks stay raw in the pipeline (F8Block) instead of being widened on load.
template <int KV, int D, bool RAW = false>
using BlockOf = std::conditional_t<KV == DT_MXFP4, MxBlock<D>,
                                   std::conditional_t<RAW && KV == DT_FP8, F8Block<D>, Block<D>>>;

__device__ __forceinline__ uint2 bload_raw8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, PKV_KV_LOAD_AUX));
  return make_uint2(w[0], w[1]);
}

// The loads of load_block<DT_FP8, D, false>, without the widening.
template <int D>
__device__ __forceinline__ void load_block_f8(F8Block<D>& b, const char* __restrict__ pool, const PageWindow& win,
                                              int t, int log2P, int64_t kv_stride_b, int64_t head_off_b,
                                              LaneOffsets lo) {
  const int P = 1 << log2P;
  const int32_t page = page_of(win, t >> log2P);
  const uint32_t slot0 = uint32_t(t & (P - 1));
  const uint32_t tile_bytes = uint32_t(P) * D;
  const char* K = uniform_ptr(pool + int64_t(page) * 2 * kv_stride_b + head_off_b);
  const auto rk = tile_rsrc(K, tile_bytes);
  const auto rv = tile_rsrc(K + kv_stride_b, tile_bytes);
  const uint32_t ks = slot0 * 32, vs = slot0 * D;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const uint32_t kj = __builtin_amdgcn_readfirstlane(ks + uint32_t(j * 32) * P);
    b.ka[j] = bload_raw8(rk, lo.k, kj);
    b.kb[j] = bload_raw8(rk, lo.k + 16 * 32, kj);
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    b.v[dt] = bload_raw8(rv, lo.v, __builtin_amdgcn_readfirstlane(vs + uint32_t(16 * BT * dt)));
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint2 w) {
  Frag8 f;
  f.w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false));
  f.w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true));
  f.w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false));
  f.w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true));
  return f.v;
}

// `n` bytes (4, 8, 16 or 32) at voff + soff of a tile, as words.
template <int N>
__device__ __forceinline__ void bload_words(uint32_t* w, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (N == 2) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, PKV_KV_LOAD_AUX);
  } else if constexpr (N == 4) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, PKV_KV_LOAD_AUX);
  } else if constexpr (N == 8) {
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, PKV_KV_LOAD_AUX));
    w[0] = v[0];
    w[1] = v[1];
  } else {
#pragma unroll
    for (int h = 0; h < N / 16; ++h) {
      const u32x4 v =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * h, soff, PKV_KV_LOAD_AUX));
#pragma unroll
      for (int i = 0; i < 4; ++i) w[4 * h + i] = v[i];
    }
  }
}

// Issue the loads of the MXFP4 block starting at token t (a multiple of 32) of a
// sequence; its page id comes from the window (which must hold it).  Eight loads:
// K codes of tokens m and 16 + m (D/8 bytes each), their scales (D/32 bytes each), the
// lane's V codes and V scales (D/4 bytes each).
template <int D>
__device__ __forceinline__ void load_block_mx(MxBlock<D>& b, const char* __restrict__ pool, const PageWindow& win,
                                              int t, int log2P, int64_t kv_stride_b, int64_t head_off_b,
                                              int lane) {
  const int P = 1 << log2P;
  const int32_t page = page_of(win, t >> log2P);
  const uint32_t slot0 = uint32_t(t & (P - 1));
  const uint32_t tb = uint32_t(tile_bytes(DT_MXFP4, P, D));
  const char* K = uniform_ptr(pool + int64_t(page) * 2 * kv_stride_b + head_off_b);
  const auto rk = tile_rsrc(K, tb);
  const auto rv = tile_rsrc(K + kv_stride_b, tb);
  const uint32_t m = lane & 15, c = lane >> 4;
  const uint32_t codes = uint32_t(P) * (D / 2);  // scales follow the codes
  const uint32_t kso = __builtin_amdgcn_readfirstlane(slot0 * (D / 2));
  bload_words<D / 8>(b.ka, rk, m * (D / 2) + c * (D / 8), kso);
  bload_words<D / 8>(b.kb, rk, (16 + m) * (D / 2) + c * (D / 8), kso);
  const uint32_t sso = __builtin_amdgcn_readfirstlane(codes + slot0 * (D / 32));
  bload_words<D / 32>(&b.ksa, rk, m * (D / 32), sso);
  bload_words<D / 32>(&b.ksb, rk, (16 + m) * (D / 32), sso);
  const uint32_t sb = slot0 >> 5;
  bload_words<D / 4>(b.v, rv, (4 * m + c) * (D / 4), __builtin_amdgcn_readfirstlane(sb * 16 * D));
  bload_words<D / 4>(b.vs, rv, c * (D / 4), __builtin_amdgcn_readfirstlane(codes + sb * D));
}

// E8M0 scale byte e as the scale operand of the scaled FP4 conversions: they read only
// the exponent field of their float scale (measured: 1.5 acts as 1.0, and +0.0 and the
// subnormals as 2^-127), so the float whose exponent field is e stands for 2^(e - 127)
// for every byte the encoder writes (0..254) -- one shift instead of an ldexp.
__device__ __forceinline__ float e8m0_operand(uint32_t e) { return __uint_as_float(e << 23); }

// Eight E2M1 codes (nibble i = element i) times `scale`, as bf16; exact, since an E2M1
// value times a power of two is a bf16 value (subnormal ones included).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float scale) {
  Frag8 f;
  f.w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  f.w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  f.w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  f.w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return f.v;
}

// An MXFP4 block decoded for the products: K exactly (code x block scale, bf16), V
// codes unscaled (their scales differ along the tokens of a lane, the contraction
// index, so they are applied to the softmax weights instead: O += (P * X_j) . V_j for
// each 32-dim block j), and the V scale bytes.
template <int D>
struct MxReady {
  bf16x8 ka[D / 32], kb[D / 32];
  bf16x8 v[D / 16];
  uint32_t vs[D / 16];
};

template <int D>
__device__ __forceinline__ const Block<D>& ready(const Block<D>& b) { return b; }

template <int D>
__device__ __forceinline__ Block<D> ready(const F8Block<D>& b) {
  Block<D> r;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    r.ka[j] = fp8x8_to_bf16(b.ka[j]);
    r.kb[j] = fp8x8_to_bf16(b.kb[j]);
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) r.v[dt] = fp8x8_to_bf16(b.v[dt]);
  return r;
}

template <int D>
__device__ __forceinline__ MxReady<D> ready(const MxBlock<D>& b) {
  MxReady<D> r;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    r.ka[j] = fp4x8_to_bf16(b.ka[j], e8m0_operand((b.ksa >> (8 * j)) & 255u));
    r.kb[j] = fp4x8_to_bf16(b.kb[j], e8m0_operand((b.ksb >> (8 * j)) & 255u));
  }
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    r.v[u] = fp4x8_to_bf16(b.v[u], 1.0f);
    r.vs[u] = b.vs[u];
  }
  return r;
}

// Online-softmax state of one wave: running max m of the raw scores q.k (per row
// lane), the lane's share of the running sum of exp2((z - m) * scale) and the output
// accumulator O [16 rows x D] (lane (n, c) holds rows 4c..4c+3 of dim 16*dt + n in
// O[dt]).  m starts at a large finite negative value rather than -inf: a row whose
// scores so far are all masked (-inf) then gets weight exp2(-inf) = 0 with no special
// case, and keeps l = 0.
constexpr float kMInit = -1e30f;

template <int D>
struct State {
  float m, l;
  f32x4 o[D / 16];
};

template <int D>
__device__ __forceinline__ void state_init(State<D>& st) {
  st.m = kMInit;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// 2^x on the hardware exponential unit (results below the normal range flush to 0,
// which for softmax weights below 2^-126 of the row maximum is what the sum keeps).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Natural-log log-sum-exp of a row from its state: m * scale (log2 units) + log2 l;
// -inf when the row saw no key.
__device__ __forceinline__ float row_lse(float m, float l, float scale) {
  return l > 0.f ? (m * scale + __log2f(l)) * kLn2 : -INFINITY;
}

// Q^T operand of a 16-row tile for kv head g: tile row n = (query j = n / G, head
// g*G + n % G); lane (n, c) holds dims 32i + 8c .. +7 of that query head, zero for rows
// with j >= nq (the sequence's queries in this call; 1 for decode).  q0 = packed row of
// the sequence's query 0.  Queries are bf16.
template <int D, int G>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[D / 32], const void* __restrict__ q, int q0, int nq,
                                       int Hq, int g, int lane) {
  const int n = lane & 15, c = lane >> 4;
  if (n / G < nq) {
    const uint16_t* base = static_cast<const uint16_t*>(q) + (int64_t(q0 + n / G) * Hq + g * G + n % G) * D + 8 * c;
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

// Merge the n partial records of one (sequence, kv head) -- record i is rec(i) --
// into the final output and log-sum-exp: LSE_h = log sum_i exp(lse_ih),
// out_h = sum_i exp(lse_ih - LSE_h) o_ih.  A record holds ROWS tile rows (row R = query
// R / G of the sequence, head g*G + R % G; rows of queries >= nq are skipped) x D.
// One workgroup of NT threads: every thread owns float4 chunks of the record (one row
// each) and a stride of records, and keeps a running (max, sum of weights, weighted
// sum) over them.  It loads its records kMergeBatch at a time, every load of a batch
// issued before any is used (the loads past the last record repeat it and are not
// used), so a batch costs one memory round trip; the record-parallel states are then
// combined in LDS.  Every thread of the workgroup must call it (it may hold barriers);
// it may be called repeatedly.
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 4;

template <int D, int G, int ROWS, int NT, typename RecFn>
__device__ __forceinline__ void merge_partials(const AttnArgs& a, int q0, int nq, int g, int n, RecFn rec) {
  constexpr int C = ROWS * D / 4;               // float4 chunks per record
  constexpr int CC = C < NT ? C : NT;           // chunk lanes
  constexpr int RP = NT / CC;                   // record-parallel factor
  constexpr int CPT = (C + NT - 1) / NT;        // chunks per thread
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
  constexpr int KB = kMergeBatch;
  for (int i0 = rp; i0 < n; i0 += KB * RP) {
    float x[KB][CPT];
    float4 o[KB][CPT];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int64_t r = rec(min(i0 + u * RP, n - 1));
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int e = min((cl + k * CC) * 4, ROWS * D - 4);  // chunks past the record: unused
        x[u][k] = a.ws_lse[r * ROWS + e / D];
        o[u][k] = *reinterpret_cast<const float4*>(a.ws_o + r * (ROWS * D) + e);
      }
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (i0 + u * RP >= n) break;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int e = (cl + k * CC) * 4;
        // rows of queries past the sequence's, and pieces that saw no key of the row
        if (e >= ROWS * D || (e / D) / G >= nq || x[u][k] == -INFINITY) continue;
        const float mn = fmaxf(m[k], x[u][k]);
        const float sa = __expf(m[k] - mn), sb = __expf(x[u][k] - mn);  // m = -inf: sa = 0
        acc[k].x = acc[k].x * sa + o[u][k].x * sb;
        acc[k].y = acc[k].y * sa + o[u][k].y * sb;
        acc[k].z = acc[k].z * sa + o[u][k].z * sb;
        acc[k].w = acc[k].w * sa + o[u][k].w * sb;
        w[k] = w[k] * sa + sb;
        m[k] = mn;
      }
    }
  }
  if constexpr (RP > 1) {
    __shared__ float4 s_acc[RP][CC * CPT];
    __shared__ float s_m[RP][CC * CPT], s_w[RP][CC * CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      s_acc[rp][cl + k * CC] = acc[k];
      s_m[rp][cl + k * CC] = m[k];
      s_w[rp][cl + k * CC] = w[k];
    }
    __syncthreads();
    if (rp == 0) {
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
    __syncthreads();  // the LDS states may be rewritten by the next call
  }
  if (rp == 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int e = (cl + k * CC) * 4;
      const int R = e / D;
      if (e < ROWS * D && R / G < nq) {
        const int d = e % D;
        const int64_t row = int64_t(q0 + R / G) * a.num_q_heads + g * G + R % G;
        const float inv = 1.f / w[k];
        uint16_t* o = static_cast<uint16_t*>(a.out) + row * D + d;
        const uint32_t lo = f32_to_bf16(acc[k].x * inv) | (f32_to_bf16(acc[k].y * inv) << 16);
        const uint32_t hi = f32_to_bf16(acc[k].z * inv) | (f32_to_bf16(acc[k].w * inv) << 16);
        *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
        if (a.lse_out && d == 0) a.lse_out[row] = m[k] + __logf(w[k]);
      }
    }
  }
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

// Raw scores^T q.k of one block for one tile of 16 query rows: lane (n, c) gets row
// n's scores of block tokens tok_of(c, e), e = 0..7.
template <int D, typename Blk>
__device__ __forceinline__ void block_scores(const Blk& b, const bf16x8 (&qf)[D / 32], float (&sc)[8]) {
  f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    sa = mma(b.ka[j], qf[j], sa);
    sb = mma(b.kb[j], qf[j], sb);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = sa[i];
    sc[4 + i] = sb[i];
  }
}

// Zero the V entries of block tokens at or past `nvalid` (slots past a range or a
// sequence may hold anything, NaN included; a zero weight alone would not cancel it).
template <int D>
__device__ __forceinline__ void mask_v_tail(Block<D>& b, int nvalid, int lane) {
  const int c = lane >> 4;
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

// Raw FP8 blocks: the same zeroing on the codes (code 0 widens to +0).
template <int D>
__device__ __forceinline__ void mask_v_tail(F8Block<D>& b, int nvalid, int lane) {
  const int c = lane >> 4;
  uint32_t keep[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (tok_of(c, e) < nvalid) keep[e >> 2] |= 0xffu << (8 * (e & 3));
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    b.v[dt].x &= keep[0];
    b.v[dt].y &= keep[1];
  }
}

// MXFP4 blocks need no V masking: codes are always finite, and the weight of a masked
// key is exactly 0, which its scale (ldexp) keeps at 0 whatever the scale byte holds.
template <int D>
__device__ __forceinline__ void mask_v_tail(MxBlock<D>&, int, int) {}

// Maximum of x over the four lanes of a score row (lanes n, n+16, n+32, n+48), in all
// four: two lane swaps across 32 and 16 lanes (no LDS permute, no lane arithmetic).
// The swaps' results are copied out of their vector before the bit casts: a bit cast
// applied to an element of that vector type reads element 0 whatever the index.
// max2 is the median of (a, b, +inf): one v_med3 with no quieting of its inputs, which
// fmaxf needs in IEEE mode for values the compiler cannot prove canonical (lane swaps,
// matrix-core results).  Scores reaching it are finite or -inf (masked), never NaN.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, __builtin_inff()); }

__device__ __forceinline__ float max8(const float (&x)[8]) {
  float m = max2(x[0], x[1]);
#pragma unroll
  for (int e = 2; e < 8; ++e) m = fmaxf(m, x[e]);
  return m;
}

__device__ __forceinline__ float row_max4(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // x[l mod 32] | x[32 + l mod 32]
  const uint32_t a0 = a[0], a1 = a[1];
  const float y = max2(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const uint32_t v = __builtin_bit_cast(uint32_t, y);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // rows 2k | 2k+1
  const uint32_t b0 = b[0], b1 = b[1];
  return max2(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}

// Online-softmax update with this block's raw (masked: -inf) scores, then O += P . V.
// `scale` turns raw scores into log2 units (softmax scale x log2 e, x the K dequant
// scale for FP8 caches); it is positive, so maxima of raw scores are maxima of the
// scaled ones and the scaling folds into one FMA per score.  A row keeps its
// reference maximum m until a block's maximum exceeds it by more than
// kRescaleLog2 (log2 units): weights up to 2^kRescaleLog2 are exact enough in fp32
// and bf16 alike, l and O always share the reference, and O is rescaled only on the
// rare blocks that move some row's reference.
constexpr float kRescaleLog2 = 8.f;

// O += P . V for one block: P (the weights p of the lane's 8 keys, fp32) packed to bf16.
template <int D>
__device__ __forceinline__ void pv_product(f32x4 (&o)[D / 16], const float (&p)[8], const Block<D>& b) {
  Frag8 pa;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    pa.w[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2 * w], p[2 * w + 1]}, bf16x2));
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = mma(pa.v, b.v[dt], o[dt]);
}

// MXFP4: for each 32-dim block j the weights carry the V scales of their keys,
// p * 2^(E - 127) (ldexp: exact, and 0 stays 0), then multiply the unscaled codes of
// the block's two 16-dim tiles.
template <int D>
__device__ __forceinline__ void pv_product(f32x4 (&o)[D / 16], const float (&p)[8], const MxReady<D>& b) {
  constexpr int J = D / 32;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    Frag8 pa;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float x[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = 2 * w + h, byte = e * J + j;
        const int ex = int((b.vs[byte >> 2] >> (8 * (byte & 3))) & 255u) - 127;
        x[h] = __builtin_ldexpf(p[e], ex);
      }
      pa.w[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2));
    }
    o[2 * j] = mma(pa.v, b.v[2 * j], o[2 * j]);
    o[2 * j + 1] = mma(pa.v, b.v[2 * j + 1], o[2 * j + 1]);
  }
}

template <int D, typename Blk>
__device__ __forceinline__ void softmax_pv(State<D>& st, const Blk& b, const float (&sc)[8],
                                           float scale, int lane) {
  const int c = lane >> 4;
  const float bm = row_max4(max8(sc));
  const bool grow = (bm - st.m) * scale > kRescaleLog2;  // same in the 4 lanes of a row
  const float mref = grow ? bm : st.m;
  const float off = -mref * scale;
  float p[8], ps = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = fast_exp2(__builtin_fmaf(sc[e], scale, off));
    ps += p[e];
  }
  if (__ballot(grow)) {  // some row moved its reference: rescale its l and O
    const float alpha = fast_exp2((st.m - mref) * scale);  // 1 for rows that did not move
    st.l *= alpha;
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * c + i, 64);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.o[dt][i] *= al[i];
    st.m = mref;
  }
  st.l += ps;
  pv_product<D>(st.o, p, b);
}

// row_max4 of NT tiles' rows, each step issued for every tile before the next step: the
// tiles' dependent chains (eight-value maximum, two lane swaps, two maxima) interleave
// instead of running one after the other.
template <int NT>
__device__ __forceinline__ void row_max4_n(const float (&sc)[NT][8], float (&out)[NT]) {
  uint32_t u[NT], a0[NT], a1[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) u[r] = __builtin_bit_cast(uint32_t, max8(sc[r]));
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const auto a = __builtin_amdgcn_permlane32_swap(u[r], u[r], false, false);
    a0[r] = a[0];
    a1[r] = a[1];
  }
#pragma unroll
  for (int r = 0; r < NT; ++r)
    u[r] = __builtin_bit_cast(uint32_t, max2(__builtin_bit_cast(float, a0[r]), __builtin_bit_cast(float, a1[r])));
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const auto b = __builtin_amdgcn_permlane16_swap(u[r], u[r], false, false);
    a0[r] = b[0];
    a1[r] = b[1];
  }
#pragma unroll
  for (int r = 0; r < NT; ++r) out[r] = max2(__builtin_bit_cast(float, a0[r]), __builtin_bit_cast(float, a1[r]));
}

// The same update split in two for NT tiles of 16 rows that share one block, so that
// the caller can put other work (the next block's scores) between and around them.
// softmax_head: the maxima, the vote and the rare rescale of l and O (a branch);
// off[r] = -m * scale of each row's reference.  softmax_tail: the weights of the
// block (straight-line vector code), their sum into l, and the P operands pa.
template <int D, int NT>
__device__ __forceinline__ void softmax_head(State<D> (&st)[NT], const float (&sc)[NT][8], float scale,
                                             float (&off)[NT], int lane, f32x4* lsum = nullptr) {
  const int c = lane >> 4;
  bool grow[NT];
  float mref[NT];
  bool any = false;
  float bms[NT];
  row_max4_n<NT>(sc, bms);
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const float bm = bms[r];
    grow[r] = (bm - st[r].m) * scale > kRescaleLog2;
    mref[r] = grow[r] ? bm : st[r].m;
    any |= grow[r];
    off[r] = -mref[r] * scale;
  }
  if (__ballot(any)) {
#pragma unroll
    for (int r = 0; r < NT; ++r) {
      const float alpha = fast_exp2((st[r].m - mref[r]) * scale);  // 1 for rows that did not move
      st[r].l *= alpha;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * c + i, 64);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[r].o[dt][i] *= al[i];
      if (lsum)
#pragma unroll
        for (int i = 0; i < 4; ++i) lsum[r][i] *= al[i];
      st[r].m = mref[r];
    }
  }
}

// SUM = false: the caller sums the weights itself (on the matrix cores, as a column of
// P . 1 beside P . V), so l is left alone.
template <int NT, bool SUM = true, typename StateT>
__device__ __forceinline__ void softmax_tail(StateT (&st)[NT], const float (&sc)[NT][8], float scale,
                                             const float (&off)[NT], Frag8 (&pa)[NT]) {
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    float p[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(__builtin_fmaf(sc[r][e], scale, off[r]));
      if constexpr (SUM) ps += p[e];
    }
    if constexpr (SUM) st[r].l += ps;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      pa[r].w[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2 * w], p[2 * w + 1]}, bf16x2));
  }
}

// The softmax half of that update for NT tiles of 16 rows that share one block: the
// P operands of all tiles (pa), their l, and one vote for the rare rescale of O; the
// caller then runs the P.V products, and can issue other MFMAs (the next block's
// scores) around this vector work.  sc[r] holds tile r's raw (masked) scores.
template <int D, int NT>
__device__ __forceinline__ void softmax_tiles(State<D> (&st)[NT], const float (&sc)[NT][8], float scale,
                                              Frag8 (&pa)[NT], int lane) {
  const int c = lane >> 4;
  bool grow[NT];
  float mref[NT];
  bool any = false;
  float bms[NT];
  row_max4_n<NT>(sc, bms);
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const float bm = bms[r];
    grow[r] = (bm - st[r].m) * scale > kRescaleLog2;
    mref[r] = grow[r] ? bm : st[r].m;
    any |= grow[r];
    const float off = -mref[r] * scale;
    float p[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(__builtin_fmaf(sc[r][e], scale, off));
      ps += p[e];
    }
#pragma unroll
    for (int w = 0; w < 4; ++w)
      pa[r].w[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2 * w], p[2 * w + 1]}, bf16x2));
    // rescale of l by a moved reference happens below; add this block's sum after it
    if (!grow[r]) st[r].l += ps;
    else {
      st[r].l = st[r].l * fast_exp2((st[r].m - mref[r]) * scale) + ps;
    }
  }
  if (__ballot(any)) {
#pragma unroll
    for (int r = 0; r < NT; ++r) {
      const float alpha = fast_exp2((st[r].m - mref[r]) * scale);  // 1 for rows that did not move
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * c + i, 64);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[r].o[dt][i] *= al[i];
      st[r].m = mref[r];
    }
  }
}

// Blocks [b0, b1) of one (sequence, kv head), folded in order by fold(block, t0), all
// of whose pages lie in the window `win` (unused with SMALLP).  N register buffers
// rotate: while block i is folded the loads of blocks i+1 .. i+N-1 are in flight.  The
// steady state runs in rounds of N blocks (every buffer index a constant) whose
// prefetches all lie in the range and are unconditional, so each fold waits only for
// its own block's loads (a partial vmcnt), never for later prefetches; the last blocks
// take a tail whose prefetches are guarded.
template <int KV, int D, bool SMALLP, bool RAW, typename FoldFn>
__device__ __forceinline__ void pipeline_blocks(const char* __restrict__ pool, const int32_t* __restrict__ bt,
                                                const PageWindow& win, int b0, int b1, int L, int log2P,
                                                int64_t kv_stride_b, int64_t head_off_b, int lane, FoldFn& fold) {
  static_assert(!RAW || (KV == DT_FP8 && !SMALLP), "raw blocks: FP8 caches with pages of >= 32 tokens");
  constexpr int N = KV == DT_MXFP4 ? PKV_MX_DEPTH : PKV_DECODE_DEPTH;
  const LaneOffsets lo = lane_offsets<KV, D>(lane);
  auto ld = [&](BlockOf<KV, D, RAW>& b, int blk) {
    if constexpr (KV == DT_MXFP4)
      load_block_mx<D>(b, pool, win, blk << LOG2_BT, log2P, kv_stride_b, head_off_b, lane);
    else if constexpr (RAW)
      load_block_f8<D>(b, pool, win, blk << LOG2_BT, log2P, kv_stride_b, head_off_b, lo);
    else
      load_block<KV, D, SMALLP>(b, pool, bt, win, blk << LOG2_BT, L, log2P, kv_stride_b, head_off_b, lo, lane);
  };
  BlockOf<KV, D, RAW> buf[N];
  const int nb = b1 - b0;
  int i = 0;
  if (nb >= 2 * N - 1) {
#pragma unroll
    for (int k = 0; k < N - 1; ++k) ld(buf[k], b0 + k);
    for (; i + 2 * N - 1 <= nb; i += N) {
#pragma unroll
      for (int k = 0; k < N; ++k) {
        ld(buf[(k + N - 1) % N], b0 + i + k + N - 1);
        fold(buf[k], (b0 + i + k) << LOG2_BT);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < N - 1; ++k)
      if (k < nb) ld(buf[k], b0 + k);
  }
  // blocks i .. nb-1, fewer than 2N - 1; blocks i .. i+N-2 are loaded or in flight
#pragma unroll
  for (int k = 0; k < 2 * N - 1; ++k) {
    if (i + k >= nb) break;
    if (i + k + N - 1 < nb) ld(buf[(k + N - 1) % N], b0 + i + k + N - 1);
    fold(buf[k % N], (b0 + i + k) << LOG2_BT);
  }
}

// Blocks [b0, b1) of one (sequence, kv head), folded in order.  With pages of >= 32
// tokens the range is cut where it leaves a 64-page window: each piece loads its
// window, then pipelines its blocks with no table load inside the loop (a conditional
// load there would make every iteration wait for all loads in flight, prefetches
// included).  The pipeline drains once per 64 pages.
template <int KV, int D, bool SMALLP, bool RAW = false, typename FoldFn>
__device__ __forceinline__ void run_blocks(const char* __restrict__ pool, const int32_t* __restrict__ bt,
                                           int b0, int b1, int L, int log2P, int64_t kv_stride_b,
                                           int64_t head_off_b, int lane, FoldFn fold,
                                           const PageWindow* win0 = nullptr) {
  if constexpr (SMALLP) {
    const PageWindow none{0, 0};
    pipeline_blocks<KV, D, true, RAW>(pool, bt, none, b0, b1, L, log2P, kv_stride_b, head_off_b, lane, fold);
  } else {
    const int log2bp = log2P - LOG2_BT;  // blocks per page, log2
    const int npages = (L + (1 << log2P) - 1) >> log2P;
    for (int c0 = b0; c0 < b1;) {
      const int base = c0 >> log2bp;
      const int c1 = min(b1, (base + 64) << log2bp);
      PageWindow win;
      if (win0 && c0 == b0)
        win = *win0;  // the caller's window of block b0's page (base b0 >> log2bp)
      else
        load_window(win, bt, base, npages, lane);
      pipeline_blocks<KV, D, false, RAW>(pool, bt, win, c0, c1, L, log2P, kv_stride_b, head_off_b, lane, fold);
      c0 = c1;
    }
  }
}


}  // namespace
}  // namespace pkv
