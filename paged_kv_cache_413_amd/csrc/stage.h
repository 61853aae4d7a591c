// Staging of K/V blocks through LDS for the matrix-core prefill kernel (and for the
// debug export of its operands): a workgroup of NTH threads fetches one 32-token block
// of one (page, kv head) from the pool into registers, decodes it to bf16 and writes it
// into an LDS stage; every wave then reads its MFMA operands from the stage with the
// same lane map it would use on the tile in HBM.
//
// A block's page comes from its sequence's block-table row ("NVIDIA TensorRT-LLM详解：
// 架构、KV Cache、调度与部署实践", §9: logical block i of a request lives in the physical
// block its table names); a block never straddles pages (pages hold >= 32 tokens here).
//
// Stage layout (bf16, 2 * D * 32 * 2 bytes): K as D/32 chunks of [32 tokens][32 dims],
// then V as [D dims][32 positions] (position order as in the pool's V sub-block).  Every
// 64-byte row (32 dims of a token, or 32 positions of a dim) is swizzled: its 16-byte
// segment c sits at segment c ^ ((row >> 1) & 3).  An operand load reads 16 bytes per
// lane, served 8 lanes at a time from a 128-byte window of the banks; its 8 lanes read 8
// consecutive rows, and the swizzle spreads them over the whole window (measured
// conflict-free; the plain layout costs 4 extra cycles per read).
#pragma once

#include "mfma_common.h"

namespace pkv {
namespace {

// Threads of the prefill kernel's workgroup, which stage each block together (a
// multiple of the 4 SIMDs' 64-lane waves).
#ifndef PKV_PF_WAVES
#define PKV_PF_WAVES 8
#endif
constexpr int kPfWaves = PKV_PF_WAVES;
constexpr int kPfThreads = 64 * kPfWaves;

// Where the blocks of one (sequence, kv head) live: the pool, the sequence's table row,
// and byte strides of the pool (per page: 2 * kv_stride_b; this kv head: head_off_b).
struct BlockSrc {
  const char* pool;
  const int32_t* bt;
  int log2P;
  int64_t kv_stride_b, head_off_b;
};

// Byte offset, in a stage, of the 16-byte operand segment lane (n, c) reads from row n
// of a 16-row group (K: token n of a chunk's half; V: dim n of a 16-dim tile).
__device__ __forceinline__ uint32_t stage_lane_offset(int lane) {
  const int n = lane & 15, c = lane >> 4;
  return uint32_t(n * 64 + 16 * (c ^ ((n >> 1) & 3)));
}

// Codes 2w, 2w+1 (byte w) of an E2M1 word times `scale`, as two bf16 (low: code 2w).
__device__ __forceinline__ uint32_t fp4_pair_to_bf16(uint32_t codes, float scale, int w) {
  switch (w) {  // the byte select is an immediate
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  }
}

// Keep-mask of the two bf16 positions 2j, 2j+1 of the 8 positions starting at 8*seg of
// a V row, for a block whose first nvalid tokens exist (position p holds token
// tok_of(p >> 3, p & 7)).
__device__ __forceinline__ uint32_t keep_pair(int seg, int j, int nvalid) {
  return (tok_of(seg, 2 * j) < nvalid ? 0x0000ffffu : 0u) | (tok_of(seg, 2 * j + 1) < nvalid ? 0xffff0000u : 0u);
}

template <int KV, int D, int NTH>
struct Stager {
  static_assert(NTH % 64 == 0, "whole waves");
  static constexpr int NW = NTH / 64;
  static constexpr int KCHUNK = BT * 32 * 2;  // bytes of one 32-dim chunk of K in a stage
  static constexpr int KBYTES = D * BT * 2;   // K of a stage; V follows
  static constexpr int BYTES = 2 * KBYTES;
  // bf16 / FP8: 1 KiB pieces of the block's tiles (one wave-wide 16-byte load each),
  // K pieces first, spread over the waves
  static constexpr int fsz = KV == DT_FP8 ? 1 : 2;
  static constexpr int FKCHUNK = BT * 32 * fsz;
  static constexpr int KPIECES = D * BT * fsz / 1024;
  static constexpr int PIECES = 2 * KPIECES;
  static constexpr int PER_WAVE = (PIECES + NW - 1) / NW;
  static constexpr bool EVEN = PIECES % NW == 0;  // else waves past PIECES copy nothing
  // MXFP4: items of 8 codes -- K: 8 dims of a token row (with its block's scale byte);
  // V: 8 positions of a dim (with the scale words of those positions: 8 for D = 128, one
  // per position; 4 for D = 64, one per two positions)
  static constexpr int MXK = 32 * D / 8, MXV = 4 * D, MXS = D / 32 >= 4 ? 8 : 4;
  static constexpr int MXK_PER = (MXK + NTH - 1) / NTH, MXV_PER = (MXV + NTH - 1) / NTH;
  static_assert(KV != DT_MXFP4 || (MXK_PER * NTH >= MXK && MXV_PER * NTH >= MXV), "every item fetched");
  static_assert(KV == DT_MXFP4 || PER_WAVE * NW >= PIECES, "every piece fetched");

  struct RegsPlain {
    uint4 w[PER_WAVE];
  };
  struct RegsMx {
    uint32_t kw[MXK_PER], ks[MXK_PER], vw[MXV_PER];
    uint32_t vs[MXV_PER][MXS];
  };
  using Regs = std::conditional_t<KV == DT_MXFP4, RegsMx, RegsPlain>;

  // Page id of block `blk` (a scalar load: it waits on the scalar counter only, never
  // on vector loads still in flight).
  __device__ static __forceinline__ int32_t page_of_block(const BlockSrc& src, int blk) {
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    return ((const_i32_ptr)(uintptr_t)src.bt)[(blk << LOG2_BT) >> src.log2P];
  }

  // Issue this thread's loads of block `blk`.
  __device__ static __forceinline__ void fetch(Regs& r, const BlockSrc& src, int blk, int tid) {
    const int P = 1 << src.log2P;
    const int32_t page = page_of_block(src, blk);
    const uint32_t slot0 = uint32_t((blk << LOG2_BT) & (P - 1));
    const char* Kt = src.pool + int64_t(page) * 2 * src.kv_stride_b + src.head_off_b;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    if constexpr (KV == DT_MXFP4) {
      const uint32_t tb = uint32_t(tile_bytes(DT_MXFP4, P, D));
      const auto rk = tile_rsrc(Kt, tb);
      const auto rv = tile_rsrc(Kt + src.kv_stride_b, tb);
      const uint32_t codes = uint32_t(P) * (D / 2);
#pragma unroll
      for (int k = 0; k < MXK_PER; ++k) {
        const int it = tid + k * NTH;
        if (MXK % NTH != 0 && it >= MXK) break;
        const int tk = it / (D / 8), j = (it % (D / 8)) >> 2, cc = it & 3;  // token, block, 8-dim group
        const uint32_t row = slot0 + uint32_t(tk);
        r.kw[k] = __builtin_amdgcn_raw_buffer_load_b32(rk, row * (D / 2) + 4 * (cc * (D / 32) + j), 0, 0);
        r.ks[k] = __builtin_amdgcn_raw_buffer_load_b8(rk, codes + row * (D / 32) + j, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < MXV_PER; ++k) {
        const int it = tid + k * NTH;
        if (MXV % NTH != 0 && it >= MXV) break;
        const int d = it >> 2, cc = it & 3, m = d & 15, u = d >> 4;
        const uint32_t sb = slot0 >> 5;
        r.vw[k] = __builtin_amdgcn_raw_buffer_load_b32(rv, sb * 16 * D + 4 * ((4 * m + cc) * (D / 16) + u), 0, 0);
        const uint32_t so = codes + (sb * 32 + 8 * cc) * (D / 32);  // positions 8cc .. 8cc+7
#pragma unroll
        for (int h = 0; h < MXS / 4; ++h) {
          const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, so + 16 * h, 0, 0));
#pragma unroll
          for (int q = 0; q < 4; ++q) r.vs[k][4 * h + q] = v[q];
        }
      }
    } else {
      const int w = tid >> 6, lane = tid & 63;
      const uint32_t tbytes = uint32_t(P) * D * fsz;
      const auto rk = tile_rsrc(Kt, tbytes);
      const auto rv = tile_rsrc(Kt + src.kv_stride_b, tbytes);
#pragma unroll
      for (int k = 0; k < PER_WAVE; ++k) {
        const int p = w + k * NW;
        if (!EVEN && p >= PIECES) break;
        // K or V piece: decided by k alone when the K pieces split evenly over the waves
        const bool is_k = KPIECES % NW == 0 ? k * NW < KPIECES : p < KPIECES;
        u32x4 v;
        if (is_k) {
          const int off = p * 1024;
          const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t(off / FKCHUNK) * P + slot0) * 32 * fsz +
                                                             uint32_t(off % FKCHUNK));
          v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, lane * 16, so, 0));
        } else {
          const uint32_t so = __builtin_amdgcn_readfirstlane(slot0 * D * fsz + uint32_t(p - KPIECES) * 1024);
          v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane * 16, so, 0));
        }
        r.w[k] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
  }

  // Decode this thread's share of a fetched block into a stage.  In a sequence's last,
  // partial block (nvalid < 32 tokens exist) the V positions past its end are zeroed
  // (they may hold anything, NaN included, and a zero weight would not cancel a NaN),
  // so the operand reads need no tail test.
  __device__ static __forceinline__ void stash(Regs& r, char* dst, int nvalid, int tid) {
    if constexpr (KV == DT_MXFP4) {
#pragma unroll
      for (int k = 0; k < MXK_PER; ++k) {
        const int it = tid + k * NTH;
        if (MXK % NTH != 0 && it >= MXK) break;
        const int tk = it / (D / 8), j = (it % (D / 8)) >> 2, cc = it & 3;
        Frag8 f;
        f.v = fp4x8_to_bf16(r.kw[k], e8m0_operand(r.ks[k] & 255u));
        *reinterpret_cast<uint4*>(dst + j * KCHUNK + tk * 64 + 16 * (cc ^ ((tk >> 1) & 3))) = f.q;
      }
#pragma unroll
      for (int k = 0; k < MXV_PER; ++k) {
        const int it = tid + k * NTH;
        if (MXV % NTH != 0 && it >= MXV) break;
        const int d = it >> 2, cc = it & 3, j = (d >> 5) & (D / 32 - 1);
        Frag8 f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // positions 8cc + 2w, +1: each code with its own scale
          uint32_t x[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            // scale byte of position 8cc + 2w + h, block j: byte (2w + h) * D/32 + j of
            // the position's scale words.  The word index is a compile-time constant
            // (j < D/32 <= 4 only moves the byte inside the word), so the scale words
            // stay in registers: a run-time index into them would make the compiler move
            // the whole array to LDS and read it back (a 9 % slower MXFP4 prefill).
            constexpr int J = D / 32;
            const int b0 = (2 * w + h) * J;
            const uint32_t word = r.vs[k][b0 >> 2];
            x[h] = fp4_pair_to_bf16(r.vw[k], e8m0_operand((word >> (8 * ((b0 & 3) + j))) & 255u), w);
          }
          f.w[w] = (x[0] & 0xffffu) | (x[1] & 0xffff0000u);  // low half of the first, high of the second
        }
        if (nvalid < BT) {  // wave-uniform: the sequence's last, partial block
#pragma unroll
          for (int w = 0; w < 4; ++w) f.w[w] &= keep_pair(cc, w, nvalid);
        }
        *reinterpret_cast<uint4*>(dst + KBYTES + d * 64 + 16 * (cc ^ ((d >> 1) & 3))) = f.q;
      }
    } else {
      const int w = tid >> 6, lane = tid & 63;
      if (nvalid < BT) {  // wave-uniform, once per sequence
#pragma unroll
        for (int k = 0; k < PER_WAVE; ++k) {
          if (w + k * NW < KPIECES) continue;
          uint32_t wd[4] = {r.w[k].x, r.w[k].y, r.w[k].z, r.w[k].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t keep = 0;
            if constexpr (fsz == 2) {
              keep = keep_pair(lane & 3, j, nvalid);  // positions 8(lane & 3) + 2j, +1
            } else {
#pragma unroll
              for (int b = 0; b < 4; ++b) {  // position 16(lane & 1) + 4j + b
                const int pp = 16 * (lane & 1) + 4 * j + b;
                keep |= tok_of(pp >> 3, pp & 7) < nvalid ? (0xffu << (8 * b)) : 0u;
              }
            }
            wd[j] &= keep;
          }
          r.w[k] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        }
      }
#pragma unroll
      for (int k = 0; k < PER_WAVE; ++k) {
        const int p = w + k * NW;
        if (!EVEN && p >= PIECES) break;
        if constexpr (fsz == 2) {
          // a 1 KiB piece is 16 rows of 64 bytes: the lane's 16 bytes are segment
          // lane & 3 of row lane >> 2
          const uint32_t wofs = uint32_t((lane >> 2) * 64 + 16 * ((lane & 3) ^ ((lane >> 3) & 3)));
          *reinterpret_cast<uint4*>(dst + p * 1024 + wofs) = r.w[k];
        } else {
          // an FP8 piece is 32 rows of 32 codes (K: the tokens of one 32-dim chunk; V: 32
          // dims); the lane's 16 codes (row lane / 2, half lane & 1) become 32 bytes of
          // bf16, segments 2(lane & 1) and 2(lane & 1) + 1 of that row of the stage
          const int row = lane >> 1, s0 = 2 * (lane & 1), swz = (row >> 1) & 3;
          char* base = dst + (p < KPIECES ? p * KCHUNK : KBYTES + (p - KPIECES) * 32 * 64) + row * 64;
          const uint32_t wd[4] = {r.w[k].x, r.w[k].y, r.w[k].z, r.w[k].w};
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            Frag8 f;
            f.w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[2 * h], 1.0f, false));
            f.w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[2 * h], 1.0f, true));
            f.w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[2 * h + 1], 1.0f, false));
            f.w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[2 * h + 1], 1.0f, true));
            *reinterpret_cast<uint4*>(base + 16 * ((s0 + h) ^ swz)) = f.q;
          }
        }
      }
    }
  }

  // Operands read back from a stage (lk = stage_lane_offset(lane)): K of chunk j, tokens
  // 16*half + (lane & 15), dims 32j + 8*(lane >> 4) .. +7; V of dims 16*dt + (lane & 15),
  // positions 8*(lane >> 4) .. +7.
  __device__ static __forceinline__ bf16x8 k_operand(const char* stg, int j, int half, uint32_t lk) {
    Frag8 f;
    f.q = *reinterpret_cast<const uint4*>(stg + j * KCHUNK + half * 16 * 64 + lk);
    return f.v;
  }
  __device__ static __forceinline__ bf16x8 v_operand(const char* stg, int dt, uint32_t lk) {
    Frag8 f;
    f.q = *reinterpret_cast<const uint4*>(stg + KBYTES + dt * 16 * 64 + lk);
    return f.v;
  }
};

}  // namespace
}  // namespace pkv
