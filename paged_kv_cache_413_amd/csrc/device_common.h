// Device helpers shared by every kernel of libpagedkv: page addressing and element
// conversions.  gfx950 (CDNA4), wave64.
//
// Page addressing ("NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践", §9: a
// request's logical blocks map to physical blocks through its block table):
// logical token t of a sequence lives in physical page block_table[t >> log2P] at
// slot t & (P - 1).  The pool is [page][K|V][kv_head][tile], one tile of P*D elements
// per (page, K|V, kv_head):
//   K tile: [D/32][P][32]  -- 32-dim column chunks, token-major inside a chunk
//   V tile: [P/S][D][S], S = min(P, 32) -- dim-major inside sub-blocks of S slots;
//           in a 32-slot sub-block, slot r sits at position vpos(r) (below)
// Both are laid out for the matrix-core decode: a wave's load of 16 token rows x 32
// dims of K, or of 16 dims x 32 tokens of V, is one contiguous run, and the slot
// order inside a V sub-block is the order in which the score tile leaves the lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_MXFP4 = 3 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element offset of tile (page, kv, head) in the pool.
__device__ __forceinline__ int64_t tile_offset(int32_t page, int kv, int head, int num_kv_heads,
                                               int page_size, int head_dim) {
  return ((int64_t(page) * 2 + kv) * num_kv_heads + head) * int64_t(page_size) * head_dim;
}

// log2 of the V sub-block length: 32 slots, or the whole page when it is shorter.
// First key a query at position pos attends to: 0, or under a limited attention window
// of W tokens the oldest of the W newest positions up to its own.
__host__ __device__ __forceinline__ int window_lo(int pos, int W) {
  return W > 0 ? (pos - W + 1 > 0 ? pos - W + 1 : 0) : 0;
}

__host__ __device__ __forceinline__ int v_sub_log2(int log2P) { return log2P < 5 ? log2P : 5; }

// Position of slot r (0..31) inside a 32-slot V sub-block: slots 4c..4c+3 go to
// positions 8c..8c+3 and slots 16+4c..16+4c+3 to 8c+4..8c+7 (c = 0..3).
__host__ __device__ __forceinline__ int vpos(int r) {
  return 8 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3);
}

// Element offset of element (t, d) of kv head `head` of the sequence whose table row
// is bt; kv = 0 (K) or 1 (V).
__device__ __forceinline__ int64_t elem_offset(const int32_t* __restrict__ bt, int t, int log2P,
                                               int kv, int head, int num_kv_heads, int head_dim,
                                               int d) {
  const int32_t page = bt[t >> log2P];
  const int slot = t & ((1 << log2P) - 1);
  const int64_t tile = tile_offset(page, kv, head, num_kv_heads, 1 << log2P, head_dim);
  if (kv == 0) return tile + ((int64_t(d >> 5) << log2P) + slot) * 32 + (d & 31);
  const int ls = v_sub_log2(log2P);
  const int r = slot & ((1 << ls) - 1);
  return tile + ((int64_t(slot >> ls) * head_dim + d) << ls) + (ls == 5 ? vpos(r) : r);
}

__device__ __forceinline__ int dtype_bytes(int dt) { return dt == DT_F32 ? 4 : (dt == DT_BF16 ? 2 : 1); }

// Bytes of one (page, K|V, kv head) tile.  MXFP4: P*D/2 code bytes, then P*D/32 scales.
__host__ __device__ __forceinline__ int64_t tile_bytes(int dt, int P, int D) {
  const int64_t n = int64_t(P) * D;
  return dt == DT_F32 ? 4 * n : dt == DT_BF16 ? 2 * n : dt == DT_FP8 ? n : n / 2 + n / 32;
}

// ---- OCP MXFP4 tiles -------------------------------------------------------------------
// Offsets inside an MXFP4 tile of P slots x D dims (see the cache description in
// paged_kv.h).  K: slot t's row of D/2 code bytes holds dims 32j + 8c + e (e = 0..7) in
// the 4-byte word c*(D/32) + j, nibble e; K scales [P][D/32] follow the codes.  V:
// 32-slot sub-blocks of 16*D code bytes; dim 16u + m of the slot at position
// k = 8c + e = vpos(slot % 32) is nibble e of word (4m + c)*(D/16) + u; V scales
// [P/32][32 positions][D/32] follow the codes.  These are the lane layouts of the
// matrix-core operands: a lane's K codes for one token are one 16-byte run (D = 128),
// and its V codes for all dims it holds are one 32-byte run.
__host__ __device__ __forceinline__ int64_t mx_k_word(int slot, int d, int D) {
  return int64_t(slot) * (D / 2) + ((((d >> 3) & 3) * (D / 32) + (d >> 5)) << 2);
}
__host__ __device__ __forceinline__ int64_t mx_v_byte(int slot, int d, int D) {
  const int k = vpos(slot & 31), c = k >> 3, e = k & 7, m = d & 15, u = d >> 4;
  return int64_t(slot >> 5) * (16 * D) + ((4 * m + c) * (D / 16) + u) * 4 + (e >> 1);
}
__host__ __device__ __forceinline__ int64_t mx_k_scale(int P, int slot, int j, int D) {
  return int64_t(P) * (D / 2) + int64_t(slot) * (D / 32) + j;
}
__host__ __device__ __forceinline__ int64_t mx_v_scale(int P, int slot, int j, int D) {
  return int64_t(P) * (D / 2) + (int64_t(slot >> 5) * 32 + vpos(slot & 31)) * (D / 32) + j;
}

// ---- bfloat16 ------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u | ((u >> 16) & 0x8000u);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---- OCP FP8 E4M3 --------------------------------------------------------------------
// Decode two codes (bytes 0,1 when hi == false, bytes 2,3 when true) of a 32-bit word
// with gfx950's conversion, which implements the OCP E4M3 format.
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, bool hi, float& a, float& b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  f2 r = hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  a = r[0];
  b = r[1];
}

// Encode one float32 value as E4M3: round to nearest, ties to even mantissa;
// magnitudes >= 448 and infinities saturate to +-448; NaN -> S.1111.111.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;          // >= 448.0f
  if (a >= 0x3c800000u) {                              // >= 2^-6: normal E4M3
    // keep 3 of the 23 mantissa bits, rounding to nearest even; a carry moves into
    // the exponent, which is what rounding up to the next binade needs
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));                   // rebias 127 -> 7
  }
  // subnormal E4M3: code = m with value m * 2^-9, m = rint(|v| * 2^9) in [0, 8]
  // (|v| * 512 is exact; 8 is the smallest normal code, 0x08)
  const float t = __uint_as_float(a) * 512.0f;
  return sign | uint32_t(__builtin_rintf(t));
}

}  // namespace pkv
