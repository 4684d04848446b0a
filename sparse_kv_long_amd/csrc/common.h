// Device helpers shared by the gfx950 kernels: bf16 unpacking, the packed
// bf16 dot product, wavefront reductions and the order-preserving float key.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace se {

constexpr int kWave = 64;
constexpr int kPage = 16;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two bf16 in one dword: element 0 in the low half.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// c + a.lo*b.lo + a.hi*b.hi with bf16 operands and fp32 accumulation
// (v_dot2c_f32_bf16).  Products of two bf16 values are exact in fp32.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float c) {
  c = dot2(a.x, b.x, c);
  c = dot2(a.y, b.y, c);
  c = dot2(a.z, b.z, c);
  c = dot2(a.w, b.w, c);
  return c;
}

// DPP lane permutations inside a row of 16 lanes.
//   0xB1: quad_perm [1,0,3,2] (lane ^ 1)     0x4E: quad_perm [2,3,0,1] (lane ^ 2)
//   0x141: row_half_mirror (lane i <-> 7-i within 8)   0x140: row_mirror (i <-> 15-i)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// All-reduce (sum) over aligned groups of N lanes, N in {1, 2, 4, 8, 16}.
// Works for mirror pairings because every lane of a sub-group holds the same
// value after the previous steps.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<0xB1>(v);
  if constexpr (N >= 4) v += dpp<0x4E>(v);
  if constexpr (N >= 8) v += dpp<0x141>(v);
  if constexpr (N >= 16) v += dpp<0x140>(v);
  return v;
}

// All-reduce over aligned groups of N lanes for any N in {1, 2, ..., 64}.
template <int N>
__device__ __forceinline__ float group_sum_any(float v) {
  if constexpr (N <= 16) {
    return group_sum<N>(v);
  } else {
    v = group_sum<16>(v);
    v += __shfl_xor(v, 16);
    if constexpr (N == 64) v += __shfl_xor(v, 32);
    return v;
  }
}

template <int N>
__device__ __forceinline__ float group_max_any(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<0xB1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<0x4E>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<0x141>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<0x140>(v));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Max / sum over the four 16-lane rows of the wave (lanes l, l^16, l^32,
// l^48) with the row-swap moves (v_permlane32_swap exchanges rows 2-3 of its
// first operand with rows 0-1 of its second, v_permlane16_swap rows 1 and 3
// with rows 0 and 2): VALU work instead of two LDS permute round trips.
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// 16-byte load with the non-temporal hint, for data read once per call.
__device__ __forceinline__ uint4 ldnt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// A raw buffer resource over `bytes` bytes from p (dword 3: the gfx9 untyped
// 32-bit format).  With bytes = 0 every load through it returns zeros without
// a memory access, so a prefetch ring can issue a fixed number of loads per
// step (the compiler then counts them and waits for one tile at a time) and
// still read nothing past its last page.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
// 16 bytes at byte offset `off` of the resource, non-temporal.
__device__ __forceinline__ uint4 ldbuf_nt16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 8 bytes at byte offset `off` of the resource.
__device__ __forceinline__ uint2 ldbuf8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}

// Order-preserving map of an fp32 to an unsigned key: a > b  <=>  key(a) > key(b)
// for non-NaN values, with -0 taken as +0 so the two compare equal.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr float kLog2e = 1.4426950408889634f;

// Copies src[0..n) (1 <= n <= N * blockDim.x) into LDS with all of a thread's
// N loads issued before the first wait: a strided loop that stores each load
// waits for that load before issuing the next.
template <int N>
__device__ __forceinline__ void stage_i32(const int32_t* __restrict__ src, int n, int32_t* dst) {
  int32_t v[N];
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = src[min((int)threadIdx.x + k * (int)blockDim.x, n - 1)];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int i = threadIdx.x + k * blockDim.x;
    if (i < n) dst[i] = v[k];
  }
}

}  // namespace se
