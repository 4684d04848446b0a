// Quest page summaries and page scoring for gfx950.
//
// Summaries (SparseEngine Fig. 3: the summaries Quest needs are attached to
// each KV block; Table 8: 16-token pages): per physical page and KV head, the
// channel-wise min and max of the keys of the page's valid tokens, stored as
// bf16 [P, Hkv, 2, D] (row 0 min, row 1 max).
//
// Page score: each query head h bounds every logit of page p by
//   U = s * sum_c max(q_c * min_c, q_c * max_c) = s * (q+ . max + q- . min)
// with q+ = max(q, 0) and q- = min(q, 0) (exact: one term of each channel is
// 0 * finite).  Both halves are bf16 contractions over the 2D-element
// summary record, so the bounds of 16 pages x 16 heads are one matrix-core
// tile per 32 k-elements (K1 below).  The KV head's score is the max (or sum)
// of its query heads' bounds.
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "se_internal.h"

namespace se {

// ---------------------------------------------------------------------------
// K0: summaries of every valid page.  One thread per (page, head, 8 channels).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void summary_build_kernel(const uint16_t* __restrict__ k,
                                                            const int32_t* __restrict__ page_table,
                                                            const int32_t* __restrict__ seq_lens,
                                                            uint16_t* __restrict__ summ, int B, int MP, int Hkv,
                                                            int D, int64_t ps, int64_t hs, int64_t ts) {
  const int cpr = D >> 3;
  const int64_t col = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)B * MP * Hkv * cpr;
  if (col >= total) return;
  const int c8 = (int)(col % cpr);
  int64_t r = col / cpr;
  const int g = (int)(r % Hkv);
  r /= Hkv;
  const int lp = (int)(r % MP);
  const int b = (int)(r / MP);
  const int n = seq_lens[b];
  if (lp * kPage >= n) return;
  const int valid = min(kPage, n - lp * kPage);
  const int64_t pid = page_table[(int64_t)b * MP + lp];
  const uint16_t* src = k + pid * ps + (int64_t)g * hs + c8 * 8;
  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = __builtin_inff();
    mx[e] = -__builtin_inff();
  }
  auto fold = [&](const uint4& w) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mn[2 * e] = fminf(mn[2 * e], bf_lo(d[e]));
      mx[2 * e] = fmaxf(mx[2 * e], bf_lo(d[e]));
      mn[2 * e + 1] = fminf(mn[2 * e + 1], bf_hi(d[e]));
      mx[2 * e + 1] = fmaxf(mx[2 * e + 1], bf_hi(d[e]));
    }
  };
  if (valid == kPage) {
    // a full page: all 16 rows requested at once (a loop with a run-time
    // count waited for each row in turn)
    uint4 w[kPage];
#pragma unroll
    for (int t = 0; t < kPage; ++t) w[t] = ldnt16(src + t * ts);
#pragma unroll
    for (int t = 0; t < kPage; ++t) fold(w[t]);
  } else {
    for (int t = 0; t < valid; ++t) fold(ld16(src + t * ts));
  }
  uint32_t omn[4], omx[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    omn[e] = (__float_as_uint(mn[2 * e]) >> 16) | (__float_as_uint(mn[2 * e + 1]) & 0xffff0000u);
    omx[e] = (__float_as_uint(mx[2 * e]) >> 16) | (__float_as_uint(mx[2 * e + 1]) & 0xffff0000u);
  }
  uint16_t* dst = summ + (pid * Hkv + g) * 2 * D + c8 * 8;
  *reinterpret_cast<uint4*>(dst) = make_uint4(omn[0], omn[1], omn[2], omn[3]);
  *reinterpret_cast<uint4*>(dst + D) = make_uint4(omx[0], omx[1], omx[2], omx[3]);
}

hipError_t launch_build_summaries(const Layout& L, int B, int MP, const uint16_t* k, const int32_t* page_table,
                                  const int32_t* seq_lens, uint16_t* summ, hipStream_t st) {
  const int64_t total = (int64_t)B * MP * L.hkv * (L.dk / 8);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(summary_build_kernel, dim3((unsigned)blocks), dim3(256), 0, st, k, page_table, seq_lens, summ,
                     B, MP, L.hkv, L.dk, L.ps, L.hs, L.ts);
  return hipGetLastError();
}

constexpr int kMaxPagesPerWave = 512;

// ---------------------------------------------------------------------------
// Shared pieces of the scoring kernels.
// ---------------------------------------------------------------------------
// Split a dword of two bf16 into its non-positive part (for the min row) and
// its non-negative part (for the max row).
__device__ __forceinline__ void split_sign(uint32_t w, uint32_t& neg, uint32_t& pos) {
  const uint32_t s = w & 0x80008000u;
  const uint32_t m = (s >> 15) * 0xffffu;  // 0xffff in each half whose sign is set
  neg = w & m;
  pos = w & ~m;
}

__device__ __forceinline__ uint4 split_neg(const uint4& w, uint4& pos) {
  uint4 neg;
  split_sign(w.x, neg.x, pos.x);
  split_sign(w.y, neg.y, pos.y);
  split_sign(w.z, neg.z, pos.z);
  split_sign(w.w, neg.w, pos.w);
  return neg;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// min/max over the valid keys of one page for 8 channels starting at `src`.
__device__ __forceinline__ void minmax8(const uint16_t* src, int64_t ts, int valid, uint4& omn, uint4& omx) {
  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = __builtin_inff();
    mx[e] = -__builtin_inff();
  }
  auto fold = [&](const uint4& w) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mn[2 * e] = fminf(mn[2 * e], bf_lo(d[e]));
      mx[2 * e] = fmaxf(mx[2 * e], bf_lo(d[e]));
      mn[2 * e + 1] = fminf(mn[2 * e + 1], bf_hi(d[e]));
      mx[2 * e + 1] = fmaxf(mx[2 * e + 1], bf_hi(d[e]));
    }
  };
  if (valid == kPage) {
    // a full page: all 16 rows requested at once (a loop with a run-time
    // count waited for each row in turn)
    uint4 w[kPage];
#pragma unroll
    for (int t = 0; t < kPage; ++t) w[t] = ldnt16(src + t * ts);
#pragma unroll
    for (int t = 0; t < kPage; ++t) fold(w[t]);
  } else {
    for (int t = 0; t < valid; ++t) fold(ld16(src + t * ts));
  }
  omn = make_uint4(pack_bf16(mn[0], mn[1]), pack_bf16(mn[2], mn[3]), pack_bf16(mn[4], mn[5]), pack_bf16(mn[6], mn[7]));
  omx = make_uint4(pack_bf16(mx[0], mx[1]), pack_bf16(mx[2], mx[3]), pack_bf16(mx[4], mx[5]), pack_bf16(mx[6], mx[7]));
}

// ---------------------------------------------------------------------------
// K1, matrix-core kernel (Dk 64 and 128).  The page bound is a dense
// contraction,
//   score[page][h] = sum_k rec[page][k] * qq[h][k],  k < 2D,
// with rec = [min | max] (the stored summary record) and qq = [q- | q+], so
// it runs on v_mfma_f32_16x16x32_bf16: 16 pages x 16 heads x 32 k per
// instruction, fp32 accumulation of exact bf16 products.  Each wave fetches
// its records 8 lanes per record (whole 128-byte lines), stages them in its
// LDS tile and reads them back in the A layout (lane l: page l%16, k-chunk
// l/16 + 4 per k step); the output element i of lane l is page 4*(l/16)+i,
// head l%16, so the KV-head max (or sum) is a 16-lane DPP reduction.  qq
// fragments sit in registers.
// The wave that owns a request's last page rebuilds that page's summary from
// its keys with all 64 lanes (each lane one 16-byte chunk: min or max of 8
// channels over the valid tokens), stores it, and scores it from LDS.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// qq fragment of head h for k-chunk ci (8 elements): q- of channels 8ci.. for
// ci < D/8, q+ of channels 8(ci - D/8).. otherwise; zero for h >= G.
// The load is unconditional (clamped head) so that a run of these issues
// back to back instead of waiting behind an exec-masked branch.
__device__ __forceinline__ uint4 qq_chunk(const uint16_t* qrow_b, int h, int G, int D, int ci) {
  const int dc = D / 8;
  uint4 pos;
  const uint4 neg = split_neg(ld16(qrow_b + (int64_t)min(h, G - 1) * D + 8 * (ci < dc ? ci : ci - dc)), pos);
  const uint4 r = ci < dc ? neg : pos;
  return h < G ? r : make_uint4(0, 0, 0, 0);
}

template <int D, int NT, bool SUM>
__global__ __launch_bounds__(256) void quest_score_mfma_kernel(ScoreArgs a, int G, int Hkv, int64_t ps, int64_t hs,
                                                               int64_t ts, int ppw) {
  constexpr int KS = 2 * D / 32;  // k steps per 16-page tile
  constexpr int NCH = D / 4;      // 16-byte chunks per record
  __shared__ int32_t ids[4 * kMaxPagesPerWave];
  __shared__ uint4 refresh_rec[4][NCH];
  __shared__ uint4 stage_lds[4 * 16 * NCH];

  const int b = blockIdx.z, g = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int blk_start = blockIdx.x * 4 * ppw;
  const int32_t* ptrow = a.page_table + (int64_t)b * a.MP;
  const uint16_t* qrow_b = a.q + ((int64_t)b * a.Hq + (int64_t)g * G) * D;
  const int col = lane & 15, kq = lane >> 4;  // A: page slot / B: head; k-chunk quarter

  // The request's length, q and the block's page ids are requested together
  // (the ids over the block's nominal range within the row: entries past the
  // request's pages are staged but never read), so the first records wait for
  // one memory round trip instead of two dependent ones.
  const int n = a.seq_lens[b];
  uint4 qb[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[nt][ks] = qq_chunk(qrow_b, nt * 16 + col, G, D, kq + 4 * ks);
  auto bfrag = [&](int nt, int ks) -> uint4 { return qb[nt][ks]; };
  stage_i32<4 * kMaxPagesPerWave / 256>(ptrow + blk_start, min(4 * ppw, a.MP - blk_start), ids);
  const int P = (n + kPage - 1) / kPage;
  const bool dense = a.topk >= P;
  if (blk_start >= P) return;
  const int plast = P - 1;
  __syncthreads();

  const int start = blk_start + wave * ppw;
  int end = min(start + ppw, P);
  if (start >= end) return;
  const bool do_refresh = a.refresh && plast >= start && plast < end;
  if (dense && !do_refresh) return;
  if (a.refresh) end = min(end, plast);

  const uint16_t* summ_g0 = a.summ + (int64_t)g * 2 * D;
  const int64_t pid_stride = (int64_t)Hkv * 2 * D;
  float* srow = a.scores + ((int64_t)b * Hkv + g) * a.MP;

  // KV-head score of the 16 pages of a tile from the accumulators; lanes with
  // col == 0 store pages base + 4*kq + i (if < lim)
  auto finish = [&](const f32x4_t (&acc)[NT], int base, int lim) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bool real = nt * 16 + col < G;
        const float x = real ? acc[nt][i] : (SUM ? 0.f : -__builtin_inff());
        v = nt == 0 ? x : (SUM ? v + x : fmaxf(v, x));
      }
      v = SUM ? group_sum<16>(v) : group_max_any<16>(v);
      const int p = base + 4 * kq + i;
      if (col == 0 && p < lim) srow[p] = v * a.scale;
    }
  };

  // the refreshed last page first: its dependent chain (keys, min/max, store,
  // score) then overlaps the streaming of this wave's other pages instead of
  // trailing it
  if (do_refresh) {
    const int64_t pid = ptrow[plast];
    const int valid = n - plast * kPage;
    const int dc = D / 8;
    uint16_t* rec = a.summ + (pid * Hkv + g) * 2 * D;
    for (int ci = lane; ci < NCH; ci += 64) {
      uint4 mn, mx;
      minmax8(a.k + pid * ps + (int64_t)g * hs + 8 * (ci < dc ? ci : ci - dc), ts, valid, mn, mx);
      const uint4 v = ci < dc ? mn : mx;
      *reinterpret_cast<uint4*>(rec + 8 * ci) = v;
      refresh_rec[wave][ci] = v;
    }
    __builtin_amdgcn_wave_barrier();
    if (!dense) {
      f32x4_t acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 d = col == 0 ? refresh_rec[wave][kq + 4 * ks] : make_uint4(0, 0, 0, 0);
          acc[nt] = mfma16(d, bfrag(nt, ks), acc[nt]);
        }
      }
      finish(acc, plast, plast + 1);  // page slot 0 of the tile is the last page
    }
  }

  if (!dense && start < end) {
    const int ntile = (end - start + 15) / 16;
    // Records are fetched 8 lanes per record (one full 128-byte line per
    // lane group and instruction: lane l takes record l/8 of each half tile
    // and chunks l%8 + 8c), written to this wave's LDS tile with chunk ci of
    // page p stored at slot ci ^ p, and read back in the MFMA A layout, which
    // the swizzle makes bank-conflict free.
    constexpr int CPR = NCH / 8;  // chunks per lane per record
    uint4* tile = stage_lds + wave * 16 * NCH;
    const int r8 = lane >> 3, j8 = lane & 7;
    uint4 dA[2][CPR];
    auto load = [&](int t, uint4 (&d)[2][CPR]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = min(start + 16 * t + 8 * u + r8, end - 1);
        const uint16_t* rec = summ_g0 + (int64_t)ids[p - blk_start] * pid_stride + 8 * j8;
#pragma unroll
        for (int c = 0; c < CPR; ++c) d[u][c] = ldnt16(rec + 64 * c);
      }
    };
    auto score = [&](int t, const uint4 (&d)[2][CPR]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int pg = 8 * u + r8;
#pragma unroll
        for (int c = 0; c < CPR; ++c) tile[pg * NCH + ((j8 + 8 * c) ^ pg)] = d[u][c];
      }
      __builtin_amdgcn_wave_barrier();
      f32x4_t acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 av = tile[col * NCH + ((kq + 4 * ks) ^ col)];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16(av, bfrag(nt, ks), acc[nt]);
      }
      __builtin_amdgcn_wave_barrier();
      finish(acc, start + 16 * t, end);
    };
    // one tile at a time, no prefetch: while a wave waits for its tile the
    // CU's other eleven waves keep HBM busy.  A tile in flight per wave on
    // top of that made the bare loads of this random 512-byte-record stream
    // slower (3,072 waves: 88 against 84.5 us); the scorer itself measured
    // the same at 128K and 19.2 against 20.6 us at 32K (events)
    for (int t = 0; t < ntile; ++t) {
      load(t, dA);
      score(t, dA);
    }
  }

}

// ---------------------------------------------------------------------------
// K1 for wide records (the 576-channel MLA key: a 2304-byte record per page).
//
// Work balance: the pages to score of all (request, KV head) units form one
// sequence (unit-major); block i takes the i-th of gridDim.x equal shares, as
// segments of one or more units, so a ragged batch keeps every block equally
// busy.  The last page of each unit, whose summary is rebuilt first, is
// handled by block (unit mod gridDim.x) before its share, which is shortened
// by kRefreshPages pages per rebuild so that those blocks finish with the rest.
//
// A block has two waves; wave w owns query heads 16w .. 16w + 15 of the KV
// head, with q of those heads for all 576 channels in registers (its
// non-positive and non-negative parts are split off per k-step).  A 16-page
// tile is fetched in two steps of eight pages; in each step a wave reads four
// whole records (9 loads of 16 bytes per lane, consecutive lanes on
// consecutive chunks) and writes them to the block's LDS tile, chunk c of page
// p at slot c ^ (p & 7).  The next tile's first step is issued before the
// current tile's matrix-core work, so each wave keeps one group of four
// records in flight almost all the time.  Each wave then forms its 16 heads x
// 16 pages of bounds over the whole contraction (A = q parts, B = the tile;
// four accumulators summed in a fixed order), scales them, reduces over its
// heads in registers and across the four lane rows, and wave 1 posts its
// per-page value to LDS; after the next barrier wave 0 adds (or takes the max
// of) both and stores the 16 scores.  No partial sums cross waves, and a tile
// costs two block barriers.
//
// Measured on the MLA ragged batch (events): 42.1 us at two blocks per CU,
// 46.8 at three and 48.0 at four (more records in flight made this random
// record stream slower, not faster), 57.6 at one; 44.0 without the one-step
// prefetch, 44.2 with both steps prefetched.  The block-cooperative form it
// replaced (four waves splitting the k dimension, partial tiles summed
// through LDS, a three-tile register ring) took 45.0 us, and 42-43 us with
// its records served from the L2 instead of HBM: its time was set by its
// per-tile chain of barriers and cross-wave sums, not by the memory.
// ---------------------------------------------------------------------------
// A last-page rebuild and score counted as this many pages of a block's share
// (its chain of dependent loads takes about as long as 80 pages of streaming
// under full load; MLA ragged batch: 42.4 / 41.9 / 41.1 / 42.1 us at 48 / 64
// / 80 / 96 pages, events; rebuilding after the shares instead measured
// slower in an earlier form of this kernel)
constexpr int kRefreshPages = 80;
constexpr int kWideUnits = 256;       // units per launch (prefix sums live in LDS)
constexpr int kWideBlocksPerCU = 2;   // one wave per SIMD: more waves in flight made this record stream slower

template <int D, bool SUM>
__global__ __launch_bounds__(128) void quest_score_wide_kernel(ScoreArgs a, int G, int Hkv, int64_t ps, int64_t hs,
                                                                int64_t ts, int u0, int nunits) {
  constexpr int KS = 2 * D / 32;     // k steps per tile
  constexpr int NCH = D / 4;         // 16-byte chunks per record
  constexpr int CPL = 4 * NCH / 64;  // loads per lane per step (four whole records per wave)
  static_assert((4 * NCH) % 64 == 0 && NCH % 8 == 0 && KS % 4 == 0, "unsupported record width");
  __shared__ uint4 tile[16 * NCH];  // slots 0 .. NCH-1 also hold a rebuilt record while it is scored
  __shared__ float agg[16];
  __shared__ int64_t pre[kWideUnits + 1];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t pid_stride = (int64_t)Hkv * 2 * D;

  auto scored = [&](int u) -> int {
    const int b = (u0 + u) / Hkv;
    const int P = (a.seq_lens[b] + kPage - 1) / kPage;
    if (a.topk >= P) return 0;
    return a.refresh ? P - 1 : P;
  };
  if (wave == 0) {
    int64_t carry = 0;
    for (int c0 = 0; c0 < nunits; c0 += kWave) {
      const int u = c0 + lane;
      const int v = u < nunits ? scored(u) : 0;
      int x = v;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      if (u < nunits) pre[u] = carry + x - v;
      carry += __shfl(x, kWave - 1);
    }
    if (lane == 0) pre[nunits] = carry;
  }
  __syncthreads();
  const int64_t total = pre[nunits];
  auto cut = [&](int i) -> int64_t {
    if (!a.refresh) return total * i / gridDim.x;
    const int64_t nr = (int64_t)i * (nunits / gridDim.x) + min(i, nunits % (int)gridDim.x);
    const int64_t v = (total + (int64_t)kRefreshPages * nunits) * i / gridDim.x - (int64_t)kRefreshPages * nr;
    return v < 0 ? 0 : v > total ? total : v;
  };
  const int64_t lo = cut(blockIdx.x), hi = max(lo, cut(blockIdx.x + 1));

  // q of head 16 * wave + col, channel chunk kq + 4m (zero past G); its
  // non-positive part pairs with k-step m (min row) and its non-negative part
  // with k-step m + KS / 2 (max row), split on the fly so that q costs 72
  // registers instead of 144 and two waves fit on each SIMD
  uint4 qr[KS / 2];
  auto load_q = [&](int b, int g) {
    const int h = 16 * wave + col;
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + (int64_t)g * G + min(h, G - 1)) * D;
#pragma unroll
    for (int m = 0; m < KS / 2; ++m) {
      const uint4 v = ld16(qrow + 8 * (kq + 4 * m));
      qr[m] = h < G ? v : make_uint4(0, 0, 0, 0);
    }
  };
  // the 16 x 16 (head x page) bounds: A = q parts, B = bfrag(ks), four accumulators
  auto mma = [&](auto bfrag, f32x4_t (&acc)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KS / 2; ++m) {
      uint4 pos;
      const uint4 neg = split_neg(qr[m], pos);
      acc[(2 * m) & 3] = mfma16(neg, bfrag(m), acc[(2 * m) & 3]);
      acc[(2 * m + 1) & 3] = mfma16(pos, bfrag(m + KS / 2), acc[(2 * m + 1) & 3]);
    }
  };
  // lane (kq, col) holds heads 16w + 4kq + i on page col; returns this wave's
  // KV-head value of page col in every lane of column col
  auto head_agg = [&](const f32x4_t (&acc)[4]) -> float {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
      const float x = 16 * wave + 4 * kq + i < G ? s * a.scale : (SUM ? 0.f : -__builtin_inff());
      v = i == 0 ? x : (SUM ? v + x : fmaxf(v, x));
    }
    return SUM ? rows_sum(v) : rows_max(v);
  };
  auto post = [&](float v) {
    if (wave == 1 && kq == 0) agg[col] = v;
  };
  // after a barrier that follows post: wave 0 stores page base + col (if < lim)
  auto complete = [&](float v, float* srow, int base, int lim) {
    if (wave == 0 && kq == 0) {
      const float o = agg[col];
      if (base + col < lim) srow[base + col] = SUM ? v + o : fmaxf(v, o);
    }
  };

  // ---- last pages first: rebuild each summary from its valid keys, store it, score it
  for (int ur = blockIdx.x; a.refresh && ur < nunits; ur += gridDim.x) {
    const int b = (u0 + ur) / Hkv, g = (u0 + ur) % Hkv;
    const int n = a.seq_lens[b];
    load_q(b, g);  // with the page lookup: the rebuild's chain of dependent loads is long enough
    const int P = (n + kPage - 1) / kPage;
    if (P == 0) continue;
    const int plast = P - 1;
    const int64_t pid = a.page_table[(int64_t)b * a.MP + plast];
    const int valid = n - plast * kPage;
    const int dc = D / 8;
    uint16_t* rec = a.summ + (pid * Hkv + g) * 2 * D;
    __syncthreads();  // the previous tile or record is no longer read
    for (int ci = threadIdx.x; ci < NCH; ci += 128) {
      uint4 mn, mx;
      minmax8(a.k + pid * ps + (int64_t)g * hs + 8 * (ci < dc ? ci : ci - dc), ts, valid, mn, mx);
      const uint4 v = ci < dc ? mn : mx;
      *reinterpret_cast<uint4*>(rec + 8 * ci) = v;
      tile[ci] = v;
    }
    __syncthreads();
    if (a.topk < P) {
      f32x4_t acc[4];
      mma([&](int ks) { return col == 0 ? tile[kq + 4 * ks] : make_uint4(0, 0, 0, 0); }, acc);
      const float v = head_agg(acc);
      post(v);
      __syncthreads();
      complete(v, a.scores + ((int64_t)b * Hkv + g) * a.MP, plast, plast + 1);  // page column 0 is the last page
    }
  }

  // ---- this block's share, unit by unit ---------------------------------------
  int u = 0;
  while (u < nunits && pre[u + 1] <= lo) ++u;
  for (; u < nunits && pre[u] < hi; ++u) {
    const int64_t s0 = max(lo, pre[u]) - pre[u], s1 = min(hi, pre[u + 1]) - pre[u];
    if (s1 <= s0) continue;
    const int b = (u0 + u) / Hkv, g = (u0 + u) % Hkv;
    const int npg = (int)(s1 - s0);
    const int32_t* pt = a.page_table + (int64_t)b * a.MP + s0;
    float* srow = a.scores + ((int64_t)b * Hkv + g) * a.MP + s0;
    const uint16_t* summ_g = a.summ + (int64_t)g * 2 * D;
    // page ids in registers: lane l holds page 64 * cw + l (idc) and 64 * (cw + 1) + l (idn), clamped
    int cw = 0;
    int idc = pt[min(lane, npg - 1)], idn = pt[min(64 + lane, npg - 1)];
    load_q(b, g);
    uint4 r[CPL];
    // records 16t + 8 * step + 4 * wave + j (j < 4), clamped to the last page
    // (a repeat that is never stored); all four lie in one 64-page window
    auto issue = [&](int t, int step) {
      const int pb = 16 * t + 8 * step + 4 * wave;
      const int src = (pb >> 6) == cw ? idc : idn;
      int idj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) idj[j] = __builtin_amdgcn_readlane(src, min(pb + j, npg - 1) & 63);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int i = 64 * c + lane, j = i / NCH, ch = i % NCH;
        const int id = j == 0 ? idj[0] : j == 1 ? idj[1] : j == 2 ? idj[2] : idj[3];
        r[c] = ldnt16(summ_g + (int64_t)id * pid_stride + 8 * ch);
      }
    };
    auto stage = [&](int step) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int i = 64 * c + lane, j = i / NCH, ch = i % NCH;
        const int pg = 8 * step + 4 * wave + j;
        tile[pg * NCH + (ch ^ (pg & 7))] = r[c];
      }
    };
    // B fragment of k-step ks: chunk kq + 4ks of page col at slot (kq + 4ks) ^ (col & 7)
    // = 8 * (ks >> 1) + ((kq + 4 * (ks & 1)) ^ (col & 7)): two lane bases, immediate offsets
    const uint4* tb[2] = {tile + col * NCH + (kq ^ (col & 7)), tile + col * NCH + ((kq + 4) ^ (col & 7))};
    const int ntile = (npg + 15) / 16;
    float vprev = 0.f;
    issue(0, 0);
    for (int t = 0; t < ntile; ++t) {
      if ((t >> 2) > cw) {
        ++cw;
        idc = idn;
        idn = pt[min(64 * (cw + 1) + lane, npg - 1)];
      }
      __syncthreads();  // tile t - 1 is read by both waves, and wave 1's value of it is posted
      if (t > 0) complete(vprev, srow, 16 * (t - 1), npg);
      stage(0);
      __builtin_amdgcn_sched_barrier(0);  // step 1 lands in the registers step 0 just left
      issue(t, 1);
      stage(1);
      __syncthreads();
      if (t + 1 < ntile) issue(t + 1, 0);
      f32x4_t acc[4];
      mma([&](int ks) { return tb[ks & 1][8 * (ks >> 1)]; }, acc);
      vprev = head_agg(acc);
      post(vprev);
    }
    __syncthreads();
    complete(vprev, srow, 16 * (ntile - 1), npg);
  }
}

static int pick_ppw(int B, int Hkv, int MP) {
  // about 3072 waves: 768 blocks, the three per CU that the matrix-core
  // kernel's LDS allows, all resident at once (measured: fewer waves leave
  // HBM idle, a second round of blocks costs more than it hides), but, while
  // that still leaves 1024 waves, at least 96 pages each, so that short
  // contexts do not pay a wave's fixed costs (ids, q, ring fill) for a handful
  // of pages (measured at 32K: 23 us at 96 pages per wave against 26 us at
  // 64); at most kMaxPagesPerWave
  const int64_t pages = (int64_t)B * Hkv * MP;
  int64_t ppw = (pages + 3071) / 3072;
  const int64_t floor_ppw = (pages + 1023) / 1024 < 96 ? (pages + 1023) / 1024 : 96;
  if (ppw < floor_ppw) ppw = floor_ppw;
  ppw = (ppw + 31) / 32 * 32;
  if (ppw > kMaxPagesPerWave) ppw = kMaxPagesPerWave;
  return (int)ppw;
}

template <int D, int NT>
static hipError_t launch_mfma(const Layout& L, const ScoreArgs& a, int G, hipStream_t st) {
  const int ppw = pick_ppw(a.B, L.hkv, a.MP);
  dim3 grid((a.MP + 4 * ppw - 1) / (4 * ppw), L.hkv, a.B);
  if (a.head_sum)
    hipLaunchKernelGGL((quest_score_mfma_kernel<D, NT, true>), grid, dim3(256), 0, st, a, G, L.hkv, L.ps, L.hs, L.ts,
                       ppw);
  else
    hipLaunchKernelGGL((quest_score_mfma_kernel<D, NT, false>), grid, dim3(256), 0, st, a, G, L.hkv, L.ps, L.hs, L.ts,
                       ppw);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_wide(const Layout& L, const ScoreArgs& a, int G, hipStream_t st) {
  // units in launches of at most kWideUnits
  const int units = a.B * L.hkv;
  for (int u0 = 0; u0 < units; u0 += kWideUnits) {
    const int nu = units - u0 < kWideUnits ? units - u0 : kWideUnits;
    if (a.head_sum)
      hipLaunchKernelGGL((quest_score_wide_kernel<D, true>), dim3(256 * kWideBlocksPerCU), dim3(128), 0, st, a, G, L.hkv,
                         L.ps, L.hs, L.ts, u0, nu);
    else
      hipLaunchKernelGGL((quest_score_wide_kernel<D, false>), dim3(256 * kWideBlocksPerCU), dim3(128), 0, st, a, G,
                         L.hkv, L.ps, L.hs, L.ts, u0, nu);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quest_scores(const Layout& L, const ScoreArgs& a, hipStream_t st) {
  const int G = a.Hq / L.hkv;
  if (a.B == 0 || a.MP == 0) return hipSuccess;
  if (L.dk == 64) return G <= 16 ? launch_mfma<64, 1>(L, a, G, st) : launch_mfma<64, 2>(L, a, G, st);
  if (L.dk == 128) return G <= 16 ? launch_mfma<128, 1>(L, a, G, st) : launch_mfma<128, 2>(L, a, G, st);
  if (L.dk == 576) return launch_wide<576>(L, a, G, st);
  return hipErrorInvalidValue;
}

}  // namespace se
