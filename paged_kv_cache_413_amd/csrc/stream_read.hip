// paged_kv_stream_read: a plain streaming read of a device buffer at the decode kernels'
// launch shape (one wave per workgroup, one wave per SIMD, 16 bytes per lane per load,
// non-temporal, several loads in flight), the practical HBM-read ceiling the attention
// kernels are compared with.  Each wave folds the words it reads into one word and
// writes it to the sink, so no load can be dropped.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace pkv {
namespace {

constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void stream_read_kernel(
    const char* __restrict__ src, int64_t bytes, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x;
  const int64_t chunks = bytes >> 10;                   // 1 KiB per wave-wide load
  const int64_t per = (chunks + gridDim.x - 1) / gridDim.x;
  const int64_t c0 = int64_t(blockIdx.x) * per, c1 = c0 + per < chunks ? c0 + per : chunks;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  uint32_t acc = 0;
  int64_t c = c0;
  for (; c + kStreamUnroll <= c1; c += kStreamUnroll) {
    u32x4 v[kStreamUnroll];
    // the buffer descriptor addresses 2^31 bytes: the wave's chunk offset goes in its base
    const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + (c << 10), 0, kStreamUnroll << 10,
                                                     0x00020000);
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k)
      v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, k << 10, 2));
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; c < c1; ++c) {
    const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + (c << 10), 0, 1024, 0x00020000);
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 0, 2));
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (lane == 0) sink[blockIdx.x] = acc;
}

}  // namespace


// Each one-wave workgroup reserves a quarter of a compute unit's 160 KiB of LDS (unused),
// so that at most four share a compute unit: one wave per SIMD, as the decode kernels
// (whose registers allow no more) are placed.
constexpr size_t kStreamLdsBytes = 40 * 1024;

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int waves, hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(waves)), dim3(64), kStreamLdsBytes, st,
                     static_cast<const char*>(src), bytes, sink);
  return hipGetLastError();
}

}  // namespace pkv
