// SnapKV eviction for gfx950: window scores, votes, max-pool and compaction.
//
// What is computed (SparseEngine Table 8: "32 scoring window; pooling kernel
// 7"; Table 10: "probability-based prefill scores"; appendix Table 7: the
// causal history [i] includes the current token; Table 15 note: physical
// eviction releases KV storage).  For request b (prompt length n, L = n - W)
// and KV head g, the G*W window rows (head hh, window index i, absolute
// position L+i) have logits z_rj = s q_r . k_j over j <= L+i and are
// normalised by a softmax over that history; the vote of prefix position
// j < L is the sum of the rows' probabilities.
//
// The window x context logits are a dense contraction, so they run on the
// matrix cores: v_mfma_f32_32x32x16_bf16 on 32 keys x 32 rows x 16 channels.
// Two passes over the keys:
//   pass 1 (rows x keys, keys as the MFMA M side): each lane holds one row and
//          16 keys of a tile, so the running max and sum of 2^z per row are
//          lane-local; pass 2's blocks merge each row's partials into
//          c_r = max_r + log2(sum_r), the row's log2 normaliser.
//   pass 2 (rows as the M side): each lane holds one key and 16 rows, so the
//          vote 2^(z - c_r) summed over rows is lane-local.  Only prefix keys
//          j < L need votes and every window row sees all of them, so pass 2
//          needs no causal mask.
// Rows come in groups of up to 128 (four 32-row MFMA tiles), whose q
// fragments a wave keeps in registers.  With one row group (SnapKV's 32-row
// window and small groups) a block's four waves take different key tiles of
// one (request, KV head).  With two to eight row groups (H2O's 128-row
// window) the block's waves are the row groups and walk the same key tiles
// together, so each tile comes from HBM once and the other waves find it in
// the CU's caches (one block per row group read every key once per group,
// measured at eight times the algorithmic bytes for four groups).
// Both passes are held to two waves per SIMD, which keeps the MFMA
// accumulators in ordinary vector registers, so the next row tile's
// matrix-core chain overlaps the current one's exponentials; in the row-
// groups-as-waves form each wave also has its next key tile in flight.
#include "common.h"
#include "se_internal.h"

namespace se {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRowsPerGroup = 128;
// Pass 1 keeps a row's reference maximum while a tile's weights stay below
// 2^20 in sum (so a row's sum stays far from the fp32 range over 32K keys).
constexpr float kRowSlackSum = 1048576.0f;
constexpr int kSnapWaves = 4;     // waves per block with one row group
constexpr int kMaxRgWaves = 8;    // row groups a block can take as its waves

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Output element r (0..15) of a 32x32 MFMA tile held by lane `lane`: row
// (M index) 8*(r/4) + 4*(lane/32) + r%4, column (N index) lane%32.
__device__ __forceinline__ int mfma_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// True when request length n leaves no more candidates than the budget, so
// every position is kept and nothing needs scoring.
__device__ __forceinline__ bool nothing_dropped(const SnapArgs& a, int n) {
  int lo, hi;
  snap_candidates(a, n, lo, hi);
  return hi - lo <= a.R;
}

// Prefix columns [vlo, vhi) whose votes the selection reads: its candidates
// [lo, hi) widened by the pooling radius, cut to the prefix [0, n - W).
__device__ __forceinline__ void vote_span(const SnapArgs& a, int n, int& vlo, int& vhi) {
  int lo, hi;
  snap_candidates(a, n, lo, hi);
  const int r = a.pool / 2;
  vlo = max(lo - r, 0);
  vhi = min(hi + r, n - a.W);
}

struct SnapGeom {
  int rows;   // G*W
  int nrg;    // row groups of up to 128 rows
  bool rgw;   // the block's waves are the row groups (2 <= nrg <= kMaxRgWaves)
  int nblk;   // blocks per (request, KV head[, row group])
  int slots;  // row-stat partials per (request, KV head, row group): key-tile walkers
};

static SnapGeom snap_geom(const SnapArgs& a) {
  SnapGeom s;
  s.rows = (a.Hq / a.Hkv) * a.W;
  s.nrg = (s.rows + kRowsPerGroup - 1) / kRowsPerGroup;
  s.rgw = s.nrg >= 2 && s.nrg <= kMaxRgWaves;
  const int tiles = (a.N + 31) / 32;
  if (s.rgw) {
    const int units = a.B * a.Hkv;
    int nblk = (2048 + units * s.nrg - 1) / (units * s.nrg);  // about 2048 waves in flight
    if (nblk > tiles) nblk = tiles;
    if (nblk < 1) nblk = 1;
    s.nblk = nblk;
    s.slots = nblk;
    return s;
  }
  const int units = a.B * a.Hkv * s.nrg;
  int nblk = (512 + units - 1) / units;  // about 2048 waves in flight
  const int maxblk = (tiles + kSnapWaves - 1) / kSnapWaves;
  if (nblk > maxblk) nblk = maxblk;
  if (nblk < 1) nblk = 1;
  s.nblk = nblk;
  s.slots = nblk * kSnapWaves;
  return s;
}

int snap_row_groups(const SnapArgs& a) { return snap_geom(a).nrg; }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t snap_workspace_bytes(const SnapArgs& a) {
  const SnapGeom s = snap_geom(a);
  size_t bytes = 0;
  bytes += align256((size_t)a.B * a.Hkv * s.nrg * s.slots * kRowsPerGroup * 2 * sizeof(float));
  bytes += align256((size_t)s.nrg * a.B * a.Hkv * a.N * sizeof(float));
  bytes += align256((size_t)a.B * a.Hkv * a.N * sizeof(float));
  return bytes;
}

SnapWork snap_workspace_carve(const SnapArgs& a, void* ws) {
  const SnapGeom s = snap_geom(a);
  char* p = static_cast<char*>(ws);
  SnapWork w;
  w.row_part = reinterpret_cast<float*>(p);
  p += align256((size_t)a.B * a.Hkv * s.nrg * s.slots * kRowsPerGroup * 2 * sizeof(float));
  w.votes = reinterpret_cast<float*>(p);
  p += align256((size_t)s.nrg * a.B * a.Hkv * a.N * sizeof(float));
  w.pooled = reinterpret_cast<float*>(p);
  return w;
}

// Load the q fragments of the block's row group: frag[rt][ks] holds, for
// lane l, row rt*32 + l%32 and channels ks*16 + 8*(l/32) .. +7.
template <int D, int NRT>
__device__ __forceinline__ void load_q_frags(const SnapArgs& a, int b, int g, int rg, int rows, uint4 (&qf)[NRT][D / 16]) {
  const int lane = threadIdx.x & 63;
  const int G = a.Hq / a.Hkv;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = rg * kRowsPerGroup + rt * 32 + (lane & 31);
    const bool ok = r < rows;
    const int hh = ok ? r / a.W : 0, i = ok ? r % a.W : 0;
    const uint16_t* qrow = a.q_win + (((int64_t)b * a.Hq + g * G + hh) * a.W + i) * D + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[rt][ks] = ok ? ld16(qrow + 16 * ks) : make_uint4(0, 0, 0, 0);
  }
}

// Key fragments of tile kt: lane l holds key kt*32 + l%32 (clamped to n-1)
// and channels ks*16 + 8*(l/32) .. +7.
template <int D>
__device__ __forceinline__ void load_k_frags(const uint16_t* kbase, int kt, int n, uint4 (&kf)[D / 16]) {
  const int lane = threadIdx.x & 63;
  int key = kt * 32 + (lane & 31);
  key = key < n ? key : n - 1;
  const uint16_t* row = kbase + (int64_t)key * D + 8 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) kf[ks] = ld16(row + 16 * ks);
}

// ---------------------------------------------------------------------------
// Pass 1: partial row max / sum of 2^z (log2-domain logits).
// Grid (Hkv * nrg, B, nblk), 4 waves, wave slot = blockIdx.z*4 + wave; or
// with RGW grid (Hkv, B, nblk), nrg waves, wave = row group, slot = blockIdx.z.
// The walkers of a unit are the slowest grid dimension, so each unit has
// blocks in every dispatch round: blocks dispatched in a later round are the
// younger ones on their CUs and lose the issue arbitration (clock stamps:
// second-round blocks ended about 7% later), and a unit whose blocks all
// fell in the last round finished last.  Measured (kernel trace, 32K
// prompts): row statistics + votes 405.4 against 411.9 us for SnapKV's
// window, 1111 against 1136 us for H2O's; giving the first round's walkers
// a larger share of the key tiles measured no better.
// ---------------------------------------------------------------------------
template <int D, int NRT, bool RGW>
__global__ __launch_bounds__(RGW ? 64 * kMaxRgWaves : 256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
snap_rowstats_kernel(SnapArgs a, float* __restrict__ row_part, int nrg, int slots, int skip_kept, float scale2) {
  const int b = blockIdx.y;
  const int g = RGW ? blockIdx.x : blockIdx.x / nrg;
  const int rg = RGW ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : blockIdx.x % nrg;
  const int n = a.lens[b];
  const int L = n - a.W;
  if (L <= 0 || (skip_kept && nothing_dropped(a, n))) return;
  const int G = a.Hq / a.Hkv;
  const int rows = G * a.W;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = RGW ? (int)blockIdx.z : (int)blockIdx.z * kSnapWaves + wave;

  uint4 qf[NRT][D / 16];
  load_q_frags<D, NRT>(a, b, g, rg, rows, qf);
  // window position of this lane's row in each row tile (rows past G*W get
  // L-1 so they see only the prefix; their statistics are never read)
  int rpos[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = rg * kRowsPerGroup + rt * 32 + (lane & 31);
    rpos[rt] = r < rows ? L + r % a.W : L - 1;
  }
  float m[NRT], l[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m[rt] = -__builtin_inff();
    l[rt] = 0.f;
  }
  const uint16_t* kbase = a.k + ((int64_t)b * a.Hkv + g) * a.N * D;
  const int tiles = (n + 31) / 32;
  auto tile = [&](const uint4(&kf)[D / 16], int kt) {
    const bool edge = kt * 32 + 31 >= L;  // tile reaches the window (or the end): mask per element
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x16_t acc = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) acc = mfma32(kf[ks], qf[rt][ks], acc);
      if (!edge) {
        // the row's reference m stays put while the tile's weights 2^(z - m)
        // sum to at most 2^kRowSlack: one fused multiply-add, exponential
        // and add per key, no maximum (the first tile, where m = -inf, and a
        // logit above m + kRowSlack take the exact step below)
        float sf = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sf += __builtin_amdgcn_exp2f(fmaf(acc[r], scale2, -m[rt]));
        if (sf <= kRowSlackSum) {
          l[rt] += sf;
          continue;
        }
      }
      float z[16];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        z[r] = acc[r] * scale2;
        if (edge) {
          const int key = kt * 32 + mfma_row(r, lane);
          if (key > rpos[rt] || key >= n) z[r] = -__builtin_inff();
        }
        tmax = fmaxf(tmax, z[r]);
      }
      const float mn = fmaxf(m[rt], tmax);
      if (mn != -__builtin_inff()) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) s += __builtin_amdgcn_exp2f(z[r] - mn);
        l[rt] = l[rt] * __builtin_amdgcn_exp2f(m[rt] - mn) + s;
        m[rt] = mn;
      }
    }
  };
  if constexpr (RGW) {
    // two key-fragment sets in turn: the walker's next tile is in flight
    // while this one is reduced (past the end the last tile is fetched
    // again, a cache hit, and not used)
    uint4 ka[D / 16], kb[D / 16];
    if (slot < tiles) load_k_frags<D>(kbase, slot, n, ka);
    for (int kt = slot; kt < tiles; kt += 2 * slots) {
      load_k_frags<D>(kbase, min(kt + slots, tiles - 1), n, kb);
      tile(ka, kt);
      if (kt + slots >= tiles) break;
      load_k_frags<D>(kbase, min(kt + 2 * slots, tiles - 1), n, ka);
      tile(kb, kt + slots);
    }
  } else {
    for (int kt = slot; kt < tiles; kt += slots) {
      uint4 kf[D / 16];
      load_k_frags<D>(kbase, kt, n, kf);
      tile(kf, kt);
    }
  }
  // combine the two lane halves (same rows, other 16 keys of each tile)
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const float mo = __shfl_xor(m[rt], 32), lo = __shfl_xor(l[rt], 32);
    const float mn = fmaxf(m[rt], mo);
    float ln = 0.f;
    if (mn != -__builtin_inff())
      ln = l[rt] * __builtin_amdgcn_exp2f(m[rt] - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
    if (lane < 32) {
      float* dst = row_part + (((((int64_t)b * a.Hkv + g) * nrg + rg) * slots + slot) * kRowsPerGroup + rt * 32 + lane) * 2;
      dst[0] = mn;
      dst[1] = ln;
    }
  }
  // row tiles past NRT*32 inside the group do not exist; nothing else to write
}

// A row's log2 normaliser c = max + log2(sum) from its pass-1 partials (one
// (max, sum) pair per key-tile walker), eight pairs per memory round trip
// (clamped indices keep the loads unconditional; repeats are not counted).
__device__ __forceinline__ float row_normaliser(const float* __restrict__ row_part, const SnapArgs& a, int b, int g,
                                                int rg, int rr, int nrg, int slots) {
  const float* src = row_part + ((((int64_t)b * a.Hkv + g) * nrg + rg) * slots) * kRowsPerGroup * 2;
  float M = -__builtin_inff(), S = 0.f;
  for (int s0 = 0; s0 < slots; s0 += 8) {
    float2 ml[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ml[j] = *reinterpret_cast<const float2*>(src + ((int64_t)min(s0 + j, slots - 1) * kRowsPerGroup + rr) * 2);
    float Mn = M;
#pragma unroll
    for (int j = 0; j < 8; ++j) Mn = fmaxf(Mn, ml[j].x);
    if (Mn == -__builtin_inff()) continue;  // no key seen yet
    S = M == -__builtin_inff() ? 0.f : S * __builtin_amdgcn_exp2f(M - Mn);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      S += (s0 + j < slots && ml[j].x != -__builtin_inff()) ? ml[j].y * __builtin_amdgcn_exp2f(ml[j].x - Mn) : 0.f;
    M = Mn;
  }
  return M + __builtin_amdgcn_logf(S);
}

// ---------------------------------------------------------------------------
// Pass 2: votes of prefix keys.  Grid and waves as pass 1.
// votes layout [nrg, B, Hkv, N].
// ---------------------------------------------------------------------------
template <int D, int NRT, bool RGW>
__global__ __launch_bounds__(RGW ? 64 * kMaxRgWaves : 256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
snap_votes_kernel(SnapArgs a, const float* __restrict__ row_part, float* __restrict__ votes, int nrg, int slots,
                  int skip_kept, float scale2) {
  __shared__ float c_lds[RGW ? kMaxRgWaves : 1][kRowsPerGroup];
  const int b = blockIdx.y;
  const int g = RGW ? blockIdx.x : blockIdx.x / nrg;
  const int rg = RGW ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : blockIdx.x % nrg;
  const int n = a.lens[b];
  const int L = n - a.W;
  if (L <= 0 || (skip_kept && nothing_dropped(a, n))) return;
  const int G = a.Hq / a.Hkv;
  const int rows = G * a.W;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = RGW ? (int)blockIdx.z : (int)blockIdx.z * kSnapWaves + wave;
  // columns whose votes are needed: the whole prefix, or (when selecting)
  // the candidates plus the pooling halo
  int vlo = 0, vhi = L;
  if (skip_kept) vote_span(a, n, vlo, vhi);
  // normalisers of the block's row groups (all nrg with RGW, else its one),
  // merged here from pass 1's partials (every block of the unit repeats this
  // small merge instead of a kernel of its own)
  const int rg0 = RGW ? 0 : rg, nrg_blk = RGW ? nrg : 1;
  for (int r = threadIdx.x; r < nrg_blk * kRowsPerGroup; r += blockDim.x) {
    const int lrg = r / kRowsPerGroup, rr = r % kRowsPerGroup;
    const int gr = (rg0 + lrg) * kRowsPerGroup + rr;
    // rows past G*W get +inf so their weight 2^(z - c) is 0
    c_lds[lrg][rr] = gr < rows ? row_normaliser(row_part, a, b, g, rg0 + lrg, rr, nrg, slots) : __builtin_inff();
  }
  __syncthreads();
  const float* cw = c_lds[RGW ? rg : 0];

  uint4 qf[NRT][D / 16];
  load_q_frags<D, NRT>(a, b, g, rg, rows, qf);
  const uint16_t* kbase = a.k + ((int64_t)b * a.Hkv + g) * a.N * D;
  float* vrow = votes + (((int64_t)rg * a.B + b) * a.Hkv + g) * a.N;
  const int t0 = vlo / 32;
  const int tiles = (vhi + 31) / 32 - t0;
  // the slot's tiles in descending order: pass 1 read them ascending, so the
  // ones it read last (the likeliest still in the caches) come first
  const int kt_last = slot < tiles ? t0 + slot + (tiles - 1 - slot) / slots * slots : -1;
  auto tile = [&](const uint4(&kf)[D / 16], int kt) {
    // with the next tile in flight (below), the normalisers are read from
    // LDS at each tile rather than held in registers, which leaves room for
    // the second set of key fragments
    int lds_off = 0;
    if constexpr (RGW) asm volatile("" : "+v"(lds_off));
    const float* cwt = cw + lds_off;
    float vote = 0.f;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x16_t acc = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) acc = mfma32(qf[rt][ks], kf[ks], acc);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 c4 = *reinterpret_cast<const float4*>(&cwt[rt * 32 + 8 * r4 + 4 * (lane >> 5)]);
        vote += __builtin_amdgcn_exp2f(acc[4 * r4 + 0] * scale2 - c4.x);
        vote += __builtin_amdgcn_exp2f(acc[4 * r4 + 1] * scale2 - c4.y);
        vote += __builtin_amdgcn_exp2f(acc[4 * r4 + 2] * scale2 - c4.z);
        vote += __builtin_amdgcn_exp2f(acc[4 * r4 + 3] * scale2 - c4.w);
      }
    }
    vote += __shfl_xor(vote, 32);
    const int key = kt * 32 + lane;
    if (lane < 32 && key < L) vrow[key] = vote;
  };
  if constexpr (RGW) {
    // two key-fragment sets in turn, as in pass 1
    uint4 ka[D / 16], kb[D / 16];
    if (kt_last >= t0) load_k_frags<D>(kbase, kt_last, n, ka);
    for (int kt = kt_last; kt >= t0; kt -= 2 * slots) {
      load_k_frags<D>(kbase, max(kt - slots, t0), n, kb);
      tile(ka, kt);
      if (kt - slots < t0) break;
      load_k_frags<D>(kbase, max(kt - 2 * slots, t0), n, ka);
      tile(kb, kt - slots);
    }
  } else {
    for (int kt = kt_last; kt >= t0; kt -= slots) {
      uint4 kf[D / 16];
      load_k_frags<D>(kbase, kt, n, kf);
      tile(kf, kt);
    }
  }
}

template <int D, int NRT, bool RGW>
static hipError_t launch_votes_t(const SnapArgs& a, const SnapWork& w, const SnapGeom& s, int skip, float* votes,
                                 hipStream_t st) {
  const float scale2 = a.scale * kLog2e;
  const dim3 grid(RGW ? a.Hkv : a.Hkv * s.nrg, a.B, s.nblk);
  const dim3 block(RGW ? 64 * s.nrg : 256);
  hipLaunchKernelGGL((snap_rowstats_kernel<D, NRT, RGW>), grid, block, 0, st, a, w.row_part, s.nrg, s.slots, skip,
                     scale2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((snap_votes_kernel<D, NRT, RGW>), grid, block, 0, st, a, w.row_part, votes, s.nrg, s.slots,
                     skip, scale2);
  return hipGetLastError();
}

hipError_t launch_snap_votes(const SnapArgs& a, const SnapWork& w, bool skip_kept, float* votes_out,
                             hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const SnapGeom s = snap_geom(a);
  const int nrt = (s.nrg > 1 ? kRowsPerGroup : s.rows + 31) / 32;  // row tiles per group
  const int skip = skip_kept ? 1 : 0;
  if (s.rgw) {  // several full row groups: four row tiles per wave
    if (a.D == 128) return launch_votes_t<128, 4, true>(a, w, s, skip, votes_out, st);
    if (a.D == 64) return launch_votes_t<64, 4, true>(a, w, s, skip, votes_out, st);
    return hipErrorInvalidValue;
  }
#define SE_V(DD, RT) \
  if (a.D == DD && nrt == RT) return launch_votes_t<DD, RT, false>(a, w, s, skip, votes_out, st);
  SE_V(128, 1) SE_V(128, 2) SE_V(128, 3) SE_V(128, 4) SE_V(64, 1) SE_V(64, 2) SE_V(64, 3) SE_V(64, 4)
#undef SE_V
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Max-pool of the votes (summed over row groups).  A block of 256 threads
// pools 2048 positions, eight per thread (256 apart): it sums the row
// groups of its positions plus a halo of `radius` on each side once into LDS
// (every load of the staging issued before the first is used), then every
// thread takes the max over its positions' windows from LDS.
// ---------------------------------------------------------------------------
constexpr int kPoolThreads = 256;
constexpr int kPoolPerThread = 8;
constexpr int kPoolTile = kPoolThreads * kPoolPerThread;
constexpr int kPoolMaxRadius = kMaxPoolKernel / 2;
constexpr int kPoolStage = (kPoolTile + 2 * kPoolMaxRadius + kPoolThreads - 1) / kPoolThreads;  // loads per thread

__global__ __launch_bounds__(kPoolThreads) void maxpool_kernel(SnapArgs a, const float* __restrict__ votes,
                                                               float* __restrict__ pooled, int radius, int nrg,
                                                               int skip_kept) {
  __shared__ float sv[kPoolStage * kPoolThreads];
  const int j0 = blockIdx.x * kPoolTile;
  const int g = blockIdx.y, b = blockIdx.z;
  const int B = a.B, Hkv = a.Hkv, N = a.N;
  const int n = a.lens[b];
  const int L = n - a.W;
  // positions pooled: the whole prefix, or (when selecting) the candidates,
  // whose windows read only the columns the votes pass wrote
  int lo = 0, hi = L, vlo = 0, vhi = L;
  if (skip_kept) {
    if (nothing_dropped(a, n)) return;
    snap_candidates(a, n, lo, hi);
    vote_span(a, n, vlo, vhi);
  }
  if (j0 >= hi || j0 + kPoolTile <= lo) return;
  const int span = kPoolTile + 2 * radius;
  float v[kPoolStage];
#pragma unroll
  for (int u = 0; u < kPoolStage; ++u) {
    const int i = u * kPoolThreads + threadIdx.x;
    const int t = j0 - radius + i;
    const bool in = i < span && t >= vlo && t < vhi;
    const int tc = in ? t : vlo;  // clamped: the load is issued either way, its value dropped
    float x = 0.f;
    for (int rg = 0; rg < nrg; ++rg) x += votes[(((int64_t)rg * B + b) * Hkv + g) * N + tc];
    v[u] = in ? x : -__builtin_inff();
  }
#pragma unroll
  for (int u = 0; u < kPoolStage; ++u) sv[u * kPoolThreads + threadIdx.x] = v[u];
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kPoolPerThread; ++e) {
    const int j = j0 + e * kPoolThreads + threadIdx.x;  // consecutive lanes, consecutive positions
    if (j < lo || j >= hi) continue;
    float best = -__builtin_inff();
    const float* w = sv + e * kPoolThreads + threadIdx.x;
    for (int d = 0; d <= 2 * radius; ++d) best = fmaxf(best, w[d]);
    pooled[((int64_t)b * Hkv + g) * N + j] = best;
  }
}

hipError_t launch_maxpool(const SnapArgs& a, const float* votes, int row_groups, float* pooled, bool skip_kept,
                          hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.pool / 2 > kPoolMaxRadius) return hipErrorInvalidValue;
  dim3 grid((a.N + kPoolTile - 1) / kPoolTile, a.Hkv, a.B);
  hipLaunchKernelGGL(maxpool_kernel, grid, dim3(kPoolThreads), 0, st, a, votes, pooled, a.pool / 2, row_groups,
                     skip_kept ? 1 : 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Compaction: k_out[b][g][r] = k[b][g][kept[r]] for r < kept_len, same for v.
// One thread per 16-byte chunk of a kept row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void compact_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                      const int32_t* __restrict__ kept_idx,
                                                      const int32_t* __restrict__ kept_len, uint16_t* __restrict__ k_out,
                                                      uint16_t* __restrict__ v_out, int Hkv, int N, int D, int cap_idx,
                                                      int cap_out) {
  const int cpr = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int64_t bg = (int64_t)b * Hkv + g;
  const int r = (int)(idx / cpr), c = (int)(idx % cpr);
  if (r >= kept_len[bg]) return;
  const int src = kept_idx[bg * cap_idx + r];
  const int64_t so = (bg * N + src) * D + 8 * c;
  const int64_t dofs = (bg * cap_out + r) * D + 8 * c;
  *reinterpret_cast<uint4*>(k_out + dofs) = ld16(k + so);
  *reinterpret_cast<uint4*>(v_out + dofs) = ld16(v + so);
}

hipError_t launch_compact(const SnapArgs& a, const int32_t* kept_idx, const int32_t* kept_len, uint16_t* k_out,
                          uint16_t* v_out, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int cap_idx = a.kcap;
  const int64_t chunks = (int64_t)cap_idx * (a.D / 8);
  dim3 grid((unsigned)((chunks + 255) / 256), a.Hkv, a.B);
  hipLaunchKernelGGL(compact_kernel, grid, dim3(256), 0, st, a.k, a.v, kept_idx, kept_len, k_out, v_out, a.Hkv, a.N,
                     a.D, cap_idx, a.cap);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Re-eviction of a compacted cache: the kept rows' indices become the
// original positions those rows stand for.  One thread per kept row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void map_positions_kernel(const int32_t* __restrict__ positions,
                                                            int32_t* __restrict__ kept_idx,
                                                            const int32_t* __restrict__ kept_len, int Hkv, int N,
                                                            int kcap) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int64_t bg = (int64_t)b * Hkv + g;
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= kept_len[bg]) return;
  const int row = kept_idx[bg * kcap + r];
  kept_idx[bg * kcap + r] = positions[bg * N + row];
}

hipError_t launch_map_positions(const SnapArgs& a, const int32_t* positions, int32_t* kept_idx,
                                const int32_t* kept_len, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  dim3 grid((unsigned)((a.kcap + 255) / 256), a.Hkv, a.B);
  hipLaunchKernelGGL(map_positions_kernel, grid, dim3(256), 0, st, positions, kept_idx, kept_len, a.Hkv, a.N,
                     a.kcap);
  return hipGetLastError();
}

}  // namespace se
