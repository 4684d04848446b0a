// A plain streaming read, the yardstick for the decode step's effective
// bandwidth (and, with ordinary loads, a re-read of a cache-sized buffer): each block reads its own contiguous share of the buffer in
// order, every lane 16 bytes per load, four loads in flight, non-temporal, and
// keeps only an XOR of the words it read (stored in the one case it equals a
// fixed constant, so the loads stay).  A contiguous share per block streams faster
// on this memory system than a grid-wide stride (measured 6.8 against
// 6.1 TB/s at 8192 blocks over 1 GiB).  Built as its own library
// (libse_hbmread.so): it is measurement equipment, not part of the decode
// path.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kNeverSeen = 0x9e3779b9u;

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// NT: non-temporal loads (a buffer read once); else ordinary loads, which
// the caches keep, so a buffer small enough for the 256 MB Infinity Cache is
// served from it when read again.
template <bool NT>
__device__ __forceinline__ u32x4 load(const u32x4* p) {
  if (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                            uint32_t* __restrict__ out) {
  const int64_t share = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t end = min((int64_t)(blockIdx.x + 1) * share, n16);
  int64_t i = (int64_t)blockIdx.x * share + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * kThreads < end; i += 4 * kThreads) {
    const u32x4 a = load<NT>(p + i);
    const u32x4 b = load<NT>(p + i + kThreads);
    const u32x4 c = load<NT>(p + i + 2 * kThreads);
    const u32x4 d = load<NT>(p + i + 3 * kThreads);
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < end; i += kThreads) acc ^= fold(load<NT>(p + i));
  if (acc == kNeverSeen) out[0] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from the device buffer `buf` once with
// `blocks` blocks of 256 threads (1 to 65536) on `stream`; `out` is one
// device uint32 that is written only if the XOR of the data equals a fixed
// constant.  Returns 0, or -1 on bad arguments (nothing launched), or the
// HIP error of the launch.
extern "C" int se_hbm_read(const void* buf, int64_t bytes, int blocks, uint32_t* out, hipStream_t stream) {
  if (!buf || !out || bytes <= 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65536) return -1;
  hipLaunchKernelGGL(hbm_read_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, static_cast<const u32x4*>(buf),
                     bytes / 16, out);
  return static_cast<int>(hipGetLastError());
}

// The same read with ordinary loads: called again on a buffer that fits the
// Infinity Cache it measures the rate at which the cache feeds the compute
// dies.  Same arguments and errors as se_hbm_read.
extern "C" int se_cache_reread(const void* buf, int64_t bytes, int blocks, uint32_t* out, hipStream_t stream) {
  if (!buf || !out || bytes <= 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65536) return -1;
  hipLaunchKernelGGL(hbm_read_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, static_cast<const u32x4*>(buf),
                     bytes / 16, out);
  return static_cast<int>(hipGetLastError());
}
