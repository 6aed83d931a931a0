// ga_decode_noalloc: ga_decode for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). Its split-K partial results live in a file-scope device array
// instead of a caller workspace; everything else is ga_decode itself.
//
// Each GPU the library runs on holds its own copy of the array (at its own
// address) until the process ends. Host code never uses the array's name as
// an address: on first use on a device, hipGetSymbolAddress gives that
// device's copy, and only that pointer is handed to the kernels. The partials
// kernel writes every partial the merge kernel reads in the same call, so the
// array needs no clearing between calls; calls that overlap on one GPU share
// it and race.
#include <atomic>
#include <mutex>

#include "../../include/ga.h"
#include "ga_internal.hpp"

static_assert(GA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

// The static scratch (see above): partial (o, m, l) rows of the decode splits.
static __device__ __align__(256) unsigned char scratch[GA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's copy of ``scratch`` (the calling thread's current device),
// looked up once per device.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" ga_status ga_decode_noalloc(const ga_attn_desc* desc, const void* q, const void* k_new,
                                       const void* v_new, const void* gate, const float* q_norm_w,
                                       const float* k_norm_w, void* k_cache, void* v_cache, int32_t cache_cap,
                                       const int32_t* cache_lens, int32_t max_cache_len, void* out, void* stream) {
  // the size check comes first (it needs no device); ga_decode checks the rest
  const size_t need = ga_decode_workspace_bytes(desc, max_cache_len);
  if (need > GA_NOALLOC_SCRATCH_BYTES)
    return (ga_status)ga::report(GA_ERR_WORKSPACE,
                                 "ga_decode_noalloc: this step needs %zu bytes of partial results, the static scratch "
                                 "holds %d (use ga_decode with a workspace)", need, GA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (desc && desc->batch > 0) {
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess)
      return (ga_status)ga::report(GA_ERR_HIP, "ga_decode_noalloc: scratch lookup: %s", hipGetErrorString(e));
  }
  return ga_decode(desc, q, k_new, v_new, gate, q_norm_w, k_norm_w, k_cache, v_cache, cache_cap, cache_lens,
                   max_cache_len, ws, GA_NOALLOC_SCRATCH_BYTES, out, stream);
}
