// se_sparse_decode_noalloc: the decode step of se_sparse_decode with its
// workspace in a device array the library holds, for callers that cannot
// allocate or pass one (code under HIP graph capture that may not call
// hipMalloc, tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy, at its own address, until the process ends.  In
// host code its name is only a stand-in for the symbol: the device address of
// the current GPU's copy comes from hipGetSymbolAddress, looked up once per
// GPU (on the first call there) and kept; kernels get that address, exactly
// as they get the caller's workspace in se_sparse_decode.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/se.h"
#include "se_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // per GPU: scratch's device address once looked up
std::mutex g_lookup;

// The device address of the current GPU's scratch array; the stream, if
// given, must belong to that GPU.
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SE_EHIP;
  if (dev >= kMaxDevices) return SE_EUNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SE_EHIP;
    if (sdev != dev) return SE_EINVAL;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_lookup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SE_EHIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SE_OK;
}

}  // namespace

extern "C" int se_sparse_decode_noalloc(const se_kv_layout* layout, const se_decode_params* params, const void* q,
                                        const void* k_pages, const void* v_pages, const int32_t* page_table,
                                        void* summaries, const int32_t* seq_lens, float* out, int32_t* selected,
                                        void* stream) {
  size_t need = 0;
  int rc = se::sparse_decode_check(layout, params, q, k_pages, v_pages, page_table, summaries, seq_lens, out, &need);
  if (rc) return rc;
  if (params->batch == 0) return SE_OK;
  if (need > SE_NOALLOC_SCRATCH_BYTES) return SE_EWORKSPACE;
  void* ws = nullptr;
  rc = scratch_address((hipStream_t)stream, &ws);
  if (rc) return rc;
  // every kernel of the step writes each workspace word it reads within the
  // same call, so what an earlier call left in the array needs no clearing
  return se::sparse_decode_enqueue(layout, params, q, k_pages, v_pages, page_table, summaries, seq_lens, out, selected,
                                   ws, (hipStream_t)stream);
}
