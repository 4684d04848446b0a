// Top-k selection for gfx950: one 1024-thread block per (request, KV head).
//
// Selects the k largest of N fp32 scores, ties to the lower index, and writes
// the chosen indices in ascending order.  Used for Quest's per-KV-head page
// budget and for SnapKV's token budget (SparseEngine Table 8: Quest's
// "selected" budgets over 16-token pages; SnapKV's selected tokens after the
// 7-wide pooling).
//
// Method: scores map to order-preserving 32-bit keys held in registers (each
// thread owns KPT consecutive indices).  The bits common to every key are
// found with a block-wide AND/OR; radix passes of up to 11 bits over the rest,
// each a 2048-bin LDS histogram of the keys that still match the chosen
// prefix, find the exact k-th largest key T and how many keys equal to T must
// be taken.
// Two block-wide exclusive scans then give every thread the number of
// T-valued keys and of selected keys before it, so the selection (key > T,
// or key == T among the first `need` such keys by index) is written in index
// order without sorting.
#include "common.h"
#include "se_internal.h"

namespace se {

constexpr int kTopkThreads = 1024;

constexpr int kRadixBits = 11;                // digit width of a descent pass
constexpr int kRadixBins = 1 << kRadixBits;   // 2048 bins: two or three passes resolve fp32 scores

struct TopkShared {
  uint32_t hist[2][kRadixBins];  // alternate passes: one is counted while the other is cleared
  int wave_tot[2][kTopkThreads / kWave];
  uint32_t wave_and[kTopkThreads / kWave], wave_or[kTopkThreads / kWave];
  int digit, above, done;
};

template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, false);
}

// Inclusive prefix sum over the wave with DPP: row_shr 1, 2, 4, 8 inside each
// row of 16 lanes, then row_bcast 15 and 31 carry row totals forward.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i<0x111>(x);
  x += dpp_i<0x112>(x);
  x += dpp_i<0x114>(x);
  x += dpp_i<0x118>(x);
  x += dpp_i<0x142, 0xa>(x);
  x += dpp_i<0x143, 0xc>(x);
  return x;
}

// Exclusive prefix sum over the block (1024 threads).  `buf` alternates
// between calls so one barrier per call suffices.
__device__ __forceinline__ int block_exclusive_scan(int v, TopkShared& sm, int buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) sm.wave_tot[buf][wave] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / kWave; ++w) before += w < wave ? sm.wave_tot[buf][w] : 0;
  return before + incl - v;
}

// Block-wide AND and OR: DPP butterflies inside each row of 16 lanes, lane
// reads across the four rows, then one pass over the per-wave results.
__device__ __forceinline__ void block_and_or(uint32_t& vand, uint32_t& vor, TopkShared& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int a = (int)vand, o = (int)vor;
  a &= dpp_i<0xB1>(a);
  o |= dpp_i<0xB1>(o);
  a &= dpp_i<0x4E>(a);
  o |= dpp_i<0x4E>(o);
  a &= dpp_i<0x141>(a);
  o |= dpp_i<0x141>(o);
  a &= dpp_i<0x140>(a);
  o |= dpp_i<0x140>(o);
  a = __builtin_amdgcn_readlane(a, 0) & __builtin_amdgcn_readlane(a, 16) & __builtin_amdgcn_readlane(a, 32) &
      __builtin_amdgcn_readlane(a, 48);
  o = __builtin_amdgcn_readlane(o, 0) | __builtin_amdgcn_readlane(o, 16) | __builtin_amdgcn_readlane(o, 32) |
      __builtin_amdgcn_readlane(o, 48);
  if (lane == 0) {
    sm.wave_and[wave] = (uint32_t)a;
    sm.wave_or[wave] = (uint32_t)o;
  }
  __syncthreads();
  vand = 0xffffffffu;
  vor = 0u;
#pragma unroll
  for (int w = 0; w < kTopkThreads / kWave; ++w) {
    vand &= sm.wave_and[w];
    vor |= sm.wave_or[w];
  }
}

// A thread's KPT consecutive scores and their translations, as loaded.
template <int KPT>
struct TopkRow {
  float f[KPT];
  int32_t t[KPT];
};

// Loads entries tid*KPT .. tid*KPT + KPT-1 of a row holding `avail` entries
// (16 bytes per load where the run is whole and aligned; zeros past the row).
// Needs no selection parameters, so a caller can request it before it knows
// how many of the entries will take part.
template <int KPT>
__device__ __forceinline__ void topk_load(const float* __restrict__ row, int avail,
                                          const int32_t* __restrict__ translate, TopkRow<KPT>& r) {
  const int base = threadIdx.x * KPT;
  const bool full = base + KPT <= avail;
  if (KPT >= 4 && full && (((uintptr_t)row) & 15) == 0) {
#pragma unroll
    for (int i = 0; i < KPT; i += 4) {
      const float4 f = *reinterpret_cast<const float4*>(row + base + i);
      r.f[i] = f.x;
      r.f[i + 1] = f.y;
      r.f[i + 2] = f.z;
      r.f[i + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < KPT; ++i) r.f[i] = (base + i < avail) ? row[base + i] : 0.f;
  }
  if (translate) {
    if (KPT >= 4 && full && (((uintptr_t)translate) & 15) == 0) {
#pragma unroll
      for (int i = 0; i < KPT; i += 4) {
        const int4 t4 = *reinterpret_cast<const int4*>(translate + base + i);
        r.t[i] = t4.x;
        r.t[i + 1] = t4.y;
        r.t[i + 2] = t4.z;
        r.t[i + 3] = t4.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) r.t[i] = (base + i < avail) ? translate[base + i] : 0;
    }
  }
}

// Selection over loaded entries (see block_topk); entries at N and past are
// ignored.  out2 is written only when translations were loaded.
template <int KPT>
__device__ __forceinline__ void block_topk_loaded(const TopkRow<KPT>& r, int N, int k, int32_t* __restrict__ out,
                                                  TopkShared& sm, int32_t* __restrict__ out2, int forced_lo,
                                                  int forced_hi, int idx_base) {
  const int tid = threadIdx.x;
  const int base = tid * KPT;
  uint32_t key[KPT];
  const int32_t* tr = r.t;
  uint32_t kand = 0xffffffffu, kor = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = (base + i < N) ? float_key(r.f[i]) : 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (base + i < forced_lo || base + i >= forced_hi) key[i] = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (base + i < N) {
      kand &= key[i];
      kor |= key[i];
    }
  }
  if (tid == 0) sm.done = 0;
  for (int i = tid; i < kRadixBins; i += kTopkThreads) sm.hist[0][i] = 0;
  // bits above the highest bit where the keys differ are common to all keys;
  // the radix passes start below them (scores of one magnitude share their
  // top byte, which would otherwise funnel every key into one bin)
  block_and_or(kand, kor, sm);  // its barrier also publishes the cleared histogram
  const uint32_t diff = kand ^ kor;
  uint32_t prefix = diff ? (kand & ~(0xffffffffu >> __builtin_clz(diff))) : kand;
  uint32_t pmask = diff ? ~(0xffffffffu >> __builtin_clz(diff)) : 0xffffffffu;
  int rem = k;
  int hi = diff ? 31 - __builtin_clz(diff) : -1;
  int hb = 0;
  // Descend until the threshold bin is resolved: either every bit is fixed
  // (ties broken by index below), or the bin holds exactly the `rem` keys
  // still needed, in which case every key of the bin is taken.  Two barriers
  // per pass: after the counting, and after the scan (during which the other
  // waves clear the next pass's histogram).
#pragma unroll 1
  while (hi >= 0) {
    const int lo = hi >= kRadixBits - 1 ? hi - (kRadixBits - 1) : 0;
    const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
    uint32_t* H = sm.hist[hb];
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (base + i < N && (key[i] & pmask) == prefix) atomicAdd(&H[(key[i] >> lo) & dmask], 1u);
    __syncthreads();
    if (tid < kWave) {
      // lane t owns bins BPL*t .. BPL*t + BPL-1; a scan of the lane totals
      // finds the lane t* whose range holds the threshold, then lanes 0..31
      // take one bin of that range each (highest first) and a second scan
      // with a ballot finds the bin: two scans instead of a serial walk
      constexpr int BPL = kRadixBins / kWave;
      static_assert(BPL <= kWave, "one bin per lane in the second scan");
      const uint4* h4 = reinterpret_cast<const uint4*>(&H[BPL * tid]);
      int local = 0;
#pragma unroll
      for (int r = 0; r < BPL / 4; ++r) {
        const uint4 v = h4[r];
        local += (int)(v.x + v.y + v.z + v.w);
      }
      const int incl = wave_incl_scan(local);
      const int total = __builtin_amdgcn_readlane(incl, 63);
      const int above_t = total - incl;  // keys in bins >= BPL * (tid + 1)
      // exactly one lane holds the threshold: 0 < rem <= total
      const int ts = __builtin_ctzll(__ballot(above_t < rem && above_t + local >= rem));
      const int above_s = __builtin_amdgcn_readlane(above_t, ts);
      const int j = tid < BPL ? tid : 0;
      const int c = tid < BPL ? (int)H[BPL * ts + (BPL - 1 - j)] : 0;
      const int cum = wave_incl_scan(c);  // keys in bins BPL*ts + BPL-1-j .. BPL*ts + BPL-1
      const int js = __builtin_ctzll(__ballot(tid < BPL && above_s + cum >= rem));
      if (tid == 0) {
        const int cnt = __builtin_amdgcn_readlane(c, js);
        const int above = above_s + __builtin_amdgcn_readlane(cum, js) - cnt;
        sm.digit = BPL * ts + (BPL - 1 - js);
        sm.above = above;
        sm.done = (cnt == rem - above) ? 1 : 0;
      }
    } else {
      uint32_t* Hn = sm.hist[hb ^ 1];
      for (int i = tid - kWave; i < kRadixBins; i += kTopkThreads - kWave) Hn[i] = 0;
    }
    __syncthreads();
    prefix |= (uint32_t)sm.digit << lo;
    pmask |= dmask << lo;
    rem -= sm.above;
    if (sm.done) break;
    hi = lo - 1;
    hb ^= 1;
  }
  // selection: (key & pmask) > prefix, or == prefix among the first `rem` such
  // keys by index (all of them when the descent stopped early)
  const int need = rem;
  const bool done = sm.done;
  int ceq = 0, cgt = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (base + i < N) {
      const uint32_t km = key[i] & pmask;
      ceq += km == prefix;
      cgt += km > prefix;
    }
  }
  int eq_before = 0;
  if (!done) eq_before = block_exclusive_scan(ceq, sm, 0);  // ties at full resolution only
  const int take_eq = done ? ceq : min(max(need - eq_before, 0), ceq);
  int pos = block_exclusive_scan(cgt + take_eq, sm, 1);
  int eq_seen = eq_before;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (base + i < N) {
      const uint32_t km = key[i] & pmask;
      bool sel = km > prefix;
      if (km == prefix) {
        sel = eq_seen < need;
        ++eq_seen;
      }
      if (sel) {
        if (out2) out2[pos] = tr[i];
        out[pos++] = idx_base + base + i;
      }
    }
  }
}

// Requires 0 < k < N <= KPT * 1024.  Writes k indices (plus idx_base) into
// out[0..k) and, when `translate` is given, translate[index] into out2[0..k).
// Indices below `forced_lo` or from `forced_hi` on take the largest key, so
// they are always kept (their number must not exceed k).
template <int KPT>
__device__ __forceinline__ void block_topk(const float* __restrict__ row, int N, int k, int32_t* __restrict__ out,
                                           TopkShared& sm, const int32_t* __restrict__ translate = nullptr,
                                           int32_t* __restrict__ out2 = nullptr, int forced_lo = 0,
                                           int forced_hi = 0x7fffffff, int idx_base = 0) {
  TopkRow<KPT> r;
  topk_load<KPT>(row, N, translate, r);
  block_topk_loaded<KPT>(r, N, k, out, sm, translate ? out2 : nullptr, forced_lo, forced_hi, idx_base);
}

// ---------------------------------------------------------------------------
// Quest: pages of (b, g).  P = ceil(seq_len/16).  Forced pages: [0, s) and
// [r_lo, P) with s = min(sink, P), r_lo = max(P - recent, s); the row holds
// kk = min(cap, P) ids (cap = topk + sink + recent), ascending, padded with -1.
// ---------------------------------------------------------------------------
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_pages_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ seq_lens,
                                                                  int32_t* __restrict__ selected,
                                                                  const int32_t* __restrict__ page_table,
                                                                  int32_t* __restrict__ phys, int Hkv, int MP,
                                                                  int topk, int sink, int recent) {
  __shared__ TopkShared sm;
  const int b = blockIdx.y, g = blockIdx.x;
  const int32_t* ptrow = page_table ? page_table + (int64_t)b * MP : nullptr;
  // the request's length and the whole score row (with its page ids) are
  // requested together: the row's loads do not wait for the length
  const int n = seq_lens[b];
  TopkRow<KPT> row;
  if (topk > 0) topk_load<KPT>(scores + ((int64_t)b * Hkv + g) * MP, MP, ptrow, row);
  const int P = (n + kPage - 1) / kPage;
  const int cap = topk + sink + recent;
  const int kk = min(cap, P);
  int32_t* out = selected + ((int64_t)b * Hkv + g) * cap;
  int32_t* out2 = phys ? phys + ((int64_t)b * Hkv + g) * cap : nullptr;
  for (int i = kk + threadIdx.x; i < cap; i += blockDim.x) {
    out[i] = -1;
    if (out2) out2[i] = -1;
  }
  if (kk == P) {
    for (int i = threadIdx.x; i < P; i += blockDim.x) {
      out[i] = i;
      if (out2) out2[i] = ptrow[i];
    }
    return;
  }
  const int s_end = min(sink, P), r_lo = max(P - recent, s_end);
  const int nforced = s_end + (P - r_lo);
  if (kk == nforced) {  // no selected budget (topk = 0): the forced pages alone, no scores read
    for (int i = threadIdx.x; i < kk; i += blockDim.x) {
      const int p = i < s_end ? i : r_lo + (i - s_end);
      out[i] = p;
      if (out2) out2[i] = ptrow[p];
    }
    return;
  }
  block_topk_loaded<KPT>(row, P, kk, out, sm, ptrow ? out2 : nullptr, s_end, r_lo, 0);
}

static int pick_kpt(int n) {
  int kpt = 1;
  while (kpt * kTopkThreads < n) kpt <<= 1;
  return kpt;
}

hipError_t launch_topk_pages(int B, int Hkv, int MP, int topk, int sink, int recent, const float* scores,
                             const int32_t* seq_lens, int32_t* selected, const int32_t* page_table, int32_t* phys,
                             hipStream_t st) {
  if (B == 0) return hipSuccess;
  dim3 grid(Hkv, B);
  switch (pick_kpt(MP)) {
#define SE_K(K)                                                                                                    \
  case K:                                                                                                          \
    hipLaunchKernelGGL(topk_pages_kernel<K>, grid, dim3(kTopkThreads), 0, st, scores, seq_lens, selected,         \
                       page_table, phys, Hkv, MP, topk, sink, recent);                                             \
    break;
    SE_K(1) SE_K(2) SE_K(4) SE_K(8) SE_K(16) SE_K(32) SE_K(64)
#undef SE_K
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SnapKV and its family: positions of (b, g) by pooled vote.  With [lo, hi)
// the candidates (snap_candidates): if hi - lo <= R keep 0..n-1; else keep
// 0..lo-1, the top R of pooled[lo..hi) (ties to the lower position), and
// hi..n-1.  Output kept_idx [B, Hkv, kcap] ascending and -1 padded;
// kept_len [B, Hkv].
// ---------------------------------------------------------------------------
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void snap_select_kernel(SnapArgs a, const float* __restrict__ pooled,
                                                                   int32_t* __restrict__ kept_idx,
                                                                   int32_t* __restrict__ kept_len) {
  __shared__ TopkShared sm;
  const int b = blockIdx.y, g = blockIdx.x;
  const int n = a.lens[b];
  const int cap = a.kcap, R = a.R;
  int lo, hi;
  snap_candidates(a, n, lo, hi);
  int32_t* out = kept_idx + ((int64_t)b * a.Hkv + g) * cap;
  if (hi - lo <= R) {
    for (int i = threadIdx.x; i < cap; i += blockDim.x) out[i] = i < n ? i : -1;
    if (threadIdx.x == 0) kept_len[(int64_t)b * a.Hkv + g] = n;
    return;
  }
  const int kept = lo + R + (n - hi);
  for (int i = threadIdx.x; i < lo; i += blockDim.x) out[i] = i;
  for (int i = threadIdx.x; i < n - hi; i += blockDim.x) out[lo + R + i] = hi + i;
  for (int i = kept + threadIdx.x; i < cap; i += blockDim.x) out[i] = -1;
  if (threadIdx.x == 0) kept_len[(int64_t)b * a.Hkv + g] = kept;
  block_topk<KPT>(pooled + ((int64_t)b * a.Hkv + g) * a.N + lo, hi - lo, R, out + lo, sm, nullptr, nullptr, 0,
                  0x7fffffff, lo);
}

hipError_t launch_snap_select(const SnapArgs& a, const float* pooled, int32_t* kept_idx, int32_t* kept_len,
                              hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  dim3 grid(a.Hkv, a.B);
  switch (pick_kpt(a.N - a.W)) {
#define SE_K(K)                                                                                                   \
  case K:                                                                                                         \
    hipLaunchKernelGGL(snap_select_kernel<K>, grid, dim3(kTopkThreads), 0, st, a, pooled, kept_idx, kept_len);     \
    break;
    SE_K(1) SE_K(2) SE_K(4) SE_K(8) SE_K(16) SE_K(32) SE_K(64)
#undef SE_K
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace se
