// Device-side validation of a call's block tables, lengths and prefix sums: the
// contract the host cannot see (page ids inside the tables, device-side lengths).
//
// With PKV_DEBUG=1 in the environment every entry point first launches
// validate_kernel, which reads only block_tables, context_lens and cu_* (or the page
// pairs of a copy) and writes the call's violation bits into a flag word of the
// library's own; every kernel of the call reads that word first and returns without
// touching the pool or the outputs when it is set.  The bits are also OR-ed into a
// sticky word that paged_kv_debug_status() reports.  A call's pages are the ones its
// kernels address: a block-table row maps logical page i to a physical page, which
// must exist ("NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践", §9, the
// logical-block -> physical-block figure); several requests may name one physical
// page, but no two appended rows may land in one slot (§10: requests share the
// blocks of a common prefix, and a request appends only to blocks of its own).
#include <mutex>
#include <vector>

#include "../../include/paged_kv.h"
#include "device_common.h"
#include "internal.h"

namespace pkv {
namespace {

// [0]: the current call's bits (read by its kernels); [1]: sticky OR since the last
// clear.  One copy per device, for the life of the process.
__device__ int32_t g_debug_flags[2];

constexpr int kValThreads = 1024;

// Logical pages [first, last] a call touches for sequence s, or first > last for none.
struct PageRange {
  int first, last;
};

__device__ __forceinline__ int call_rows(const ValidateArgs& v, int s) {
  return v.cu ? v.cu[s + 1] - v.cu[s] : 1;
}

__device__ PageRange pages_of(const CacheArgs& c, const SeqArgs& sq, const ValidateArgs& v, int s, int L, int n) {
  const int lp = c.log2_page;
  if (v.kind == VK_APPEND) {
    if (n <= 0) return {1, 0};
    return {(L - n) >> lp, (L - 1) >> lp};
  }
  if (v.kind == VK_GATHER) return {0, (L - 1) >> lp};
  // attention: from the 32-token block holding the first key the call's earliest
  // query sees (window) to the page of the last key
  const int lo = window_lo(L - (v.kind == VK_PREFILL ? n : 1), sq.window);
  return {((lo >> 5) << 5) >> lp, (L - 1) >> lp};
}

__global__ __launch_bounds__(kValThreads) void validate_kernel(CacheArgs c, SeqArgs sq, ValidateArgs v,
                                                               int32_t* __restrict__ flags) {
  __shared__ int bits;
  if (threadIdx.x == 0) bits = 0;
  __syncthreads();
  int mine = 0;
  const int S = sq.num_seqs;
  if (v.kind == VK_COPY) {
    for (int i = threadIdx.x; i < v.num_pairs; i += kValThreads) {
      const int32_t s = v.src[i], d = v.dst[i];
      if (s < 0 || s >= c.num_pages || d < 0 || d >= c.num_pages) mine |= PKV_DEBUG_PAGE_RANGE;
      for (int j = 0; j < v.num_pairs; ++j)
        if (v.src[j] == d || (j != i && v.dst[j] == d)) mine |= PKV_DEBUG_COPY_PAIRS;
    }
  } else {
    if (v.cu && threadIdx.x == 0 && (v.cu[0] != 0 || v.cu[S] != v.total_rows)) mine |= PKV_DEBUG_CU;
    for (int s = threadIdx.x; s < S; s += kValThreads) {
      const int L = sq.context_lens[s];
      const int n = call_rows(v, s);
      if (n < 0) {
        mine |= PKV_DEBUG_CU;
        continue;
      }
      if (L < 1 || L > sq.max_context_len || n > L || (v.kind == VK_PREFILL && n > v.max_q_len)) {
        mine |= PKV_DEBUG_LENGTH;
        continue;  // its table entries may lie past the row: not read
      }
      const PageRange r = pages_of(c, sq, v, s, L, n);
      const int32_t* bt = sq.block_tables + int64_t(s) * sq.max_pages_per_seq;
      for (int p = r.first; p <= r.last; ++p) {
        const int32_t page = bt[p];
        if (page < 0 || page >= c.num_pages) mine |= PKV_DEBUG_PAGE_RANGE;
      }
    }
  }
  if (mine) atomicOr(&bits, mine);
  __syncthreads();
  // Appends: no two rows may name one slot.  Rows of one sequence take distinct
  // positions, so two rows share a slot only when their pages coincide: compare every
  // pair of (sequence, logical page) runs the append writes, if everything else holds.
  if (v.kind == VK_APPEND && bits == 0) {
    const int lp = c.log2_page;
    int dup = 0;
    for (int s = threadIdx.x; s < S && !dup; s += kValThreads) {
      const int L = sq.context_lens[s], n = call_rows(v, s);
      if (n <= 0) continue;
      const int32_t* bt = sq.block_tables + int64_t(s) * sq.max_pages_per_seq;
      for (int p = (L - n) >> lp; p <= (L - 1) >> lp && !dup; ++p) {
        const int32_t page = bt[p];
        const int a0 = max(L - n, p << lp) - (p << lp), a1 = min(L, (p + 1) << lp) - (p << lp);  // slots [a0, a1)
        for (int s2 = s; s2 < S && !dup; ++s2) {
          const int L2 = sq.context_lens[s2], n2 = call_rows(v, s2);
          if (n2 <= 0) continue;
          const int32_t* bt2 = sq.block_tables + int64_t(s2) * sq.max_pages_per_seq;
          for (int p2 = s2 == s ? p + 1 : (L2 - n2) >> lp; p2 <= (L2 - 1) >> lp; ++p2) {
            if (bt2[p2] != page) continue;
            const int b0 = max(L2 - n2, p2 << lp) - (p2 << lp), b1 = min(L2, (p2 + 1) << lp) - (p2 << lp);
            if (a0 < b1 && b0 < a1) {
              dup = 1;
              break;
            }
          }
        }
      }
    }
    if (dup) atomicOr(&bits, PKV_DEBUG_DUP_SLOT);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int b = bits;
    flags[0] = b;
    if (b) atomicOr(&flags[1], b);
  }
}

// Address of g_debug_flags on each device, looked up once per device.
int32_t* flags_ptr() {
  static std::mutex mu;
  static std::vector<int32_t*> ptrs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (dev >= int(ptrs.size())) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_debug_flags)) != hipSuccess) return nullptr;
    ptrs[dev] = static_cast<int32_t*>(p);
  }
  return ptrs[dev];
}

}  // namespace

hipError_t launch_validate(CacheArgs& c, const SeqArgs& s, const ValidateArgs& v, hipStream_t stream) {
  int32_t* f = flags_ptr();
  if (!f) return hipErrorInvalidSymbol;
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(kValThreads), 0, stream, c, s, v, f);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) c.debug_flag = f;
  return e;
}

hipError_t read_debug_status(bool clear, int32_t* out) {
  int32_t* f = flags_ptr();
  if (!f) return hipErrorInvalidSymbol;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  if ((e = hipMemcpy(out, f + 1, sizeof(int32_t), hipMemcpyDeviceToHost)) != hipSuccess) return e;
  if (clear) {
    const int32_t zero[2] = {0, 0};
    e = hipMemcpy(f, zero, sizeof zero, hipMemcpyHostToDevice);
  }
  return e;
}

}  // namespace pkv
