// paged_attn_decode_noalloc: paged_attn_decode with its workspace in a device array the
// library owns, for callers that cannot allocate (code under graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The array is a file-scope device variable: each device the library runs on holds its
// own copy until the process ends.  In host code its name is only a stand-in for the
// symbol, not a device address; the address of this device's copy is looked up once
// per device with hipGetSymbolAddress (the device current) and kept, and only that
// address is handed to the kernels.  The decode workspace needs no initialisation
// (every record and descriptor is written before it is read), so nothing is cleared.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/paged_kv.h"

namespace {

static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

// This device's copy of `scratch`, or NULL (with *err set) when the lookup fails.
char* scratch_ptr(hipError_t* err) {
  static std::mutex mu;
  static std::vector<char*> ptrs;
  int dev = 0;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (dev >= int(ptrs.size())) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if ((*err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return nullptr;
    ptrs[dev] = static_cast<char*>(p);
  }
  *err = hipSuccess;
  return ptrs[dev];
}

}  // namespace

namespace pkv {
int set_error(int code, const char* fmt, ...);
}

extern "C" int paged_attn_decode_noalloc(const pkv_cache_t* cache, const pkv_seqs_t* seqs, const void* q,
                                         int32_t q_dtype, int32_t num_q_heads, float sm_scale, int32_t num_splits,
                                         void* out, float* lse_out, void* stream) {
  hipError_t e;
  char* ws = scratch_ptr(&e);
  if (!ws) return pkv::set_error(PKV_ELAUNCH, "paged_attn_decode_noalloc: no address for the scratch array: %s",
                                 hipGetErrorString(e));
  // Arguments the call rejects give 0 here and are reported by the call itself.
  const size_t need = paged_attn_decode_workspace_size(cache, seqs, q_dtype, num_q_heads, num_splits);
  if (need > size_t(PKV_NOALLOC_SCRATCH_BYTES))
    return pkv::set_error(PKV_EWORKSPACE,
                          "paged_attn_decode_noalloc: this call needs %zu bytes of workspace, the library's "
                          "scratch array holds %zu (use paged_attn_decode with a workspace of your own)",
                          need, size_t(PKV_NOALLOC_SCRATCH_BYTES));
  return paged_attn_decode(cache, seqs, q, q_dtype, num_q_heads, sm_scale, num_splits, out, lse_out, ws,
                           size_t(PKV_NOALLOC_SCRATCH_BYTES), stream);
}
