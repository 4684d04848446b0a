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
// 0 * finite).  Both halves are bf16 dot products, so the score is 2D packed
// v_dot2 operations per head.  The KV head's score is the max (or sum) of
// its query heads' bounds.
//
// Work layout of the fast kernel: 8 lanes read one 2*D-element record with
// 16-byte loads (a record of D = 128 is 512 B: lanes 0-7 read chunks 0-7,
// then 8-15, ...), so one wave instruction covers 8 records; each lane owns
// the same channel chunks of the min half and the max half, keeps q+ and q-
// of those channels for all G heads in registers, and the 8 partial sums of
// a record are combined with three DPP steps.
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
  for (int t = 0; t < valid; ++t) {
    const uint4 w = ld16(src + t * ts);
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mn[2 * e] = fminf(mn[2 * e], bf_lo(d[e]));
      mx[2 * e] = fmaxf(mx[2 * e], bf_lo(d[e]));
      mn[2 * e + 1] = fminf(mn[2 * e + 1], bf_hi(d[e]));
      mx[2 * e + 1] = fmaxf(mx[2 * e + 1], bf_hi(d[e]));
    }
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
  for (int t = 0; t < valid; ++t) {
    const uint4 w = ld16(src + t * ts);
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mn[2 * e] = fminf(mn[2 * e], bf_lo(d[e]));
      mx[2 * e] = fmaxf(mx[2 * e], bf_lo(d[e]));
      mn[2 * e + 1] = fminf(mn[2 * e + 1], bf_hi(d[e]));
      mx[2 * e + 1] = fmaxf(mx[2 * e + 1], bf_hi(d[e]));
    }
  }
  omn = make_uint4(pack_bf16(mn[0], mn[1]), pack_bf16(mn[2], mn[3]), pack_bf16(mn[4], mn[5]), pack_bf16(mn[6], mn[7]));
  omx = make_uint4(pack_bf16(mx[0], mx[1]), pack_bf16(mx[2], mx[3]), pack_bf16(mx[4], mx[5]), pack_bf16(mx[6], mx[7]));
}

// ---------------------------------------------------------------------------
// K1, register kernel: G * D <= 1024 (q+ and q- of the lane's channels of all
// G heads stay in registers).  Grid (ceil(MP / (4*ppw)), Hkv, B), 4 waves per
// block, each wave scores `ppw` consecutive pages of one (request, KV head).
// With `refresh`, the wave holding the request's last page first rebuilds
// that page's summary from its keys, stores it, and scores it from the
// rebuilt values.
// ---------------------------------------------------------------------------
template <int G, int D, bool SUM>
__global__ __launch_bounds__(256) void quest_score_reg_kernel(ScoreArgs a, int Hkv, int64_t ps, int64_t hs,
                                                               int64_t ts, int ppw) {
  constexpr int LPP = 8;
  constexpr int NCH = D / 4;      // 16-byte chunks per record
  constexpr int CPL = NCH / LPP;  // chunks per lane
  constexpr int NCC = CPL / 2;    // channel chunks per lane
  constexpr int U = 2;            // pages per lane group per stage (a stage is 8*U pages)
  static_assert((D / 8) % LPP == 0, "channel chunks must split evenly over the 8 lanes of a record");
  __shared__ int32_t ids[4 * kMaxPagesPerWave];

  const int b = blockIdx.z, g = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 7, pg = lane >> 3;
  const int n = a.seq_lens[b];
  const int P = (n + kPage - 1) / kPage;
  const bool dense = a.topk >= P;
  const int blk_start = blockIdx.x * 4 * ppw;
  if (blk_start >= P) return;
  const int blk_end = min(blk_start + 4 * ppw, P);
  const int plast = P - 1;
  const int32_t* ptrow = a.page_table + (int64_t)b * a.MP;
  // stage the block's physical page ids in LDS (one coalesced pass)
  if (!dense)
    for (int i = threadIdx.x; i < blk_end - blk_start; i += blockDim.x) ids[i] = ptrow[blk_start + i];
  __syncthreads();

  const int start = blk_start + wave * ppw;
  int end = min(start + ppw, P);
  if (start >= end) return;
  const bool do_refresh = a.refresh && plast >= start && plast < end;
  if (dense && !do_refresh) return;
  if (a.refresh) end = min(end, plast);

  uint4 qn[G][NCC], qp[G][NCC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + g * G + h) * D;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) qn[h][cc] = split_neg(ld16(qrow + 8 * (j + LPP * cc)), qp[h][cc]);
  }

  const int64_t rec_stride = 2 * D;
  const uint16_t* summ_g = a.summ + (int64_t)g * rec_stride + 8 * j;
  const int64_t pid_stride = (int64_t)Hkv * rec_stride;
  float* srow = a.scores + ((int64_t)b * Hkv + g) * a.MP;

  auto page_score = [&](const uint4 (&d)[CPL]) -> float {
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc[h] = dot8(qn[h][cc], d[cc], acc[h]);
        acc[h] = dot8(qp[h][cc], d[NCC + cc], acc[h]);
      }
    }
    float r = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float v = group_sum<LPP>(acc[h]);
      r = (h == 0) ? v : (SUM ? r + v : fmaxf(r, v));
    }
    return r * a.scale;
  };

  if (!dense && start < end) {
    // Two register stages of 8*U pages: the next stage's loads are in flight
    // while the current one is scored.  Loads are unconditional (page index
    // clamped to the range; a clamped stage re-reads cached records) so that
    // no branch sits between a load and its use; only the stores are masked.
    const int nst = (end - start + 8 * U - 1) / (8 * U);
    uint4 dA[U][CPL], dB[U][CPL];
    auto load = [&](int st, uint4 (&d)[U][CPL]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = min(start + st * 8 * U + 8 * u + pg, end - 1);
        const uint16_t* rec = summ_g + (int64_t)ids[p - blk_start] * pid_stride;
#pragma unroll
        for (int c = 0; c < CPL; ++c) d[u][c] = ldnt16(rec + 8 * LPP * c);
      }
    };
    auto score = [&](int st, const uint4 (&d)[U][CPL]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = start + st * 8 * U + 8 * u + pg;
        const float sc = page_score(d[u]);
        if (p < end && j == 0) srow[p] = sc;
      }
    };
    load(0, dA);
    for (int st = 0; st < nst; st += 2) {
      load(min(st + 1, nst - 1), dB);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
      score(st, dA);
      load(min(st + 2, nst - 1), dA);
      __builtin_amdgcn_sched_barrier(0);
      score(st + 1, dB);
    }
  }

  if (do_refresh) {
    const int64_t pid = ptrow[plast];
    const int valid = n - plast * kPage;
    const uint16_t* kb = a.k + pid * ps + (int64_t)g * hs;
    uint4 d[CPL];
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) minmax8(kb + 8 * (j + LPP * cc), ts, valid, d[cc], d[NCC + cc]);
    uint16_t* rec = a.summ + (pid * Hkv + g) * rec_stride + 8 * j;
    if (pg == 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) *reinterpret_cast<uint4*>(rec + 8 * LPP * c) = d[c];
    }
    const float sc = page_score(d);
    if (!dense && lane == 0) srow[plast] = sc;
  }
}

// ---------------------------------------------------------------------------
// K1, generic kernel: any G <= 64 and D in {64, 128, 576}.  q+ and q- of all
// heads live in LDS; each lane keeps its chunks of the record in registers
// and loops over the heads.  Same grid and refresh rule as above.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void quest_score_lds_kernel(ScoreArgs a, int G, int Hkv, int64_t ps, int64_t hs,
                                                              int64_t ts, int ppw) {
  constexpr int LPP = 8;
  constexpr int NCH = D / 4;
  constexpr int CPL = NCH / LPP;
  constexpr int NCC = CPL / 2;
  constexpr int DC = D / 8;  // channel chunks per head
  static_assert(DC % LPP == 0, "channel chunks must split evenly over the 8 lanes of a record");
  extern __shared__ uint4 qs[];  // [G][DC] q-  then [G][DC] q+

  const int b = blockIdx.z, g = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 7, pg = lane >> 3;
  const int n = a.seq_lens[b];
  const int P = (n + kPage - 1) / kPage;
  const bool dense = a.topk >= P;
  uint4* qneg = qs;
  uint4* qpos = qs + G * DC;
  for (int i = threadIdx.x; i < G * DC; i += blockDim.x) {
    const int h = i / DC, c = i % DC;
    uint4 pos;
    qneg[i] = split_neg(ld16(a.q + ((int64_t)b * a.Hq + g * G + h) * D + 8 * c), pos);
    qpos[i] = pos;
  }
  __syncthreads();

  const int start = (blockIdx.x * 4 + wave) * ppw;
  int end = min(start + ppw, P);
  if (start >= end) return;
  const int plast = P - 1;
  const bool do_refresh = a.refresh && plast >= start && plast < end;
  if (dense && !do_refresh) return;
  if (a.refresh) end = min(end, plast);

  const int64_t rec_stride = 2 * D;
  const uint16_t* summ_g = a.summ + (int64_t)g * rec_stride;
  float* srow = a.scores + ((int64_t)b * Hkv + g) * a.MP;
  const int32_t* ptrow = a.page_table + (int64_t)b * a.MP;
  const bool SUM = a.head_sum != 0;

  auto page_score = [&](const uint4 (&d)[CPL]) -> float {
    float r = 0.f;
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) {
        acc = dot8(qneg[h * DC + j + LPP * cc], d[cc], acc);
        acc = dot8(qpos[h * DC + j + LPP * cc], d[NCC + cc], acc);
      }
      const float v = group_sum<LPP>(acc);
      r = (h == 0) ? v : (SUM ? r + v : fmaxf(r, v));
    }
    return r * a.scale;
  };

  if (!dense) {
    for (int p0 = start; p0 < end; p0 += 8) {
      const int p = p0 + pg;
      const bool ok = p < end;
      const int64_t pid = ok ? ptrow[p] : 0;
      uint4 d[CPL];
      const uint16_t* rec = summ_g + pid * Hkv * rec_stride + 8 * j;
#pragma unroll
      for (int c = 0; c < CPL; ++c) d[c] = ok ? ld16(rec + 8 * LPP * c) : make_uint4(0, 0, 0, 0);
      const float sc = page_score(d);
      if (ok && j == 0) srow[p] = sc;
    }
  }

  if (do_refresh) {
    const int64_t pid = ptrow[plast];
    const int valid = n - plast * kPage;
    const uint16_t* kb = a.k + pid * ps + (int64_t)g * hs;
    uint4 d[CPL];
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) minmax8(kb + 8 * (j + LPP * cc), ts, valid, d[cc], d[NCC + cc]);
    uint16_t* rec = a.summ + (pid * Hkv + g) * rec_stride + 8 * j;
    if (pg == 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) *reinterpret_cast<uint4*>(rec + 8 * LPP * c) = d[c];
    }
    const float sc = page_score(d);
    if (!dense && lane == 0) srow[plast] = sc;
  }
}

// ---------------------------------------------------------------------------
// K1, matrix-core kernel.  The page bound is a dense contraction,
//   score[page][h] = sum_k rec[page][k] * qq[h][k],  k < 2D,
// with rec = [min | max] (the stored summary record) and qq = [q- | q+], so
// it runs on v_mfma_f32_16x16x32_bf16: 16 pages x 16 heads x 32 k per
// instruction, fp32 accumulation of exact bf16 products.  Lane l supplies
// page l%16 and k-chunk l/16 (+4 per k step) of the record, i.e. 16-byte
// loads that form 64-byte contiguous runs; the output element i of lane l is
// page 4*(l/16)+i, head l%16, so the KV-head max (or sum) is a 16-lane DPP
// reduction.  qq fragments sit in registers.
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
  const int n = a.seq_lens[b];
  const int P = (n + kPage - 1) / kPage;
  const bool dense = a.topk >= P;
  const int blk_start = blockIdx.x * 4 * ppw;
  if (blk_start >= P) return;
  const int blk_end = min(blk_start + 4 * ppw, P);
  const int plast = P - 1;
  const int32_t* ptrow = a.page_table + (int64_t)b * a.MP;
  const uint16_t* qrow_b = a.q + ((int64_t)b * a.Hq + (int64_t)g * G) * D;
  const int col = lane & 15, kq = lane >> 4;  // A: page slot / B: head; k-chunk quarter

  if (!dense) stage_i32<4 * kMaxPagesPerWave / 256>(ptrow + blk_start, blk_end - blk_start, ids);
  __syncthreads();

  const int start = blk_start + wave * ppw;
  int end = min(start + ppw, P);
  if (start >= end) return;
  const bool do_refresh = a.refresh && plast >= start && plast < end;
  if (dense && !do_refresh) return;
  if (a.refresh) end = min(end, plast);

  uint4 qb[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[nt][ks] = qq_chunk(qrow_b, nt * 16 + col, G, D, kq + 4 * ks);
  auto bfrag = [&](int nt, int ks) -> uint4 { return qb[nt][ks]; };

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
    uint4 dA[2][CPR], dB[2][CPR];
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
    load(0, dA);
    for (int t = 0; t < ntile; t += 2) {
      load(min(t + 1, ntile - 1), dB);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
      score(t, dA);
      load(min(t + 2, ntile - 1), dA);
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < ntile) score(t + 1, dB);
    }
  }

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
}

// ---------------------------------------------------------------------------
// K1 for wide records (the 576-channel MLA key: a 2304-byte record per page).
// A block streams 16-page tiles: its 256 threads fetch a tile's records as
// whole contiguous runs (consecutive threads take consecutive 16-byte chunks
// of a record), write them to an LDS tile with chunk c of page p stored at
// slot c ^ (p & 7), and the four waves then split the tile's k dimension
// (wave w: k-steps 9w..9w+8 of 36), reading their A fragments from LDS
// without bank conflicts and keeping their q+/q- fragments in registers.
// The partial tiles are summed through LDS in a fixed order and wave w
// finishes rows i = w (pages 4*kq + w of the tile).
// ---------------------------------------------------------------------------
constexpr int kWidePagesPerBlock = 2048;

template <int D, int NT, int RD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void quest_score_wide_kernel(ScoreArgs a, int G, int Hkv, int64_t ps, int64_t hs, int64_t ts, int ppb) {
  constexpr int KS = 2 * D / 32;  // k steps per tile
  constexpr int KW = KS / 4;      // k steps per wave
  constexpr int NCH = D / 4;      // 16-byte chunks per record
  constexpr int CPT = 16 * NCH / 256;  // chunks per thread per tile
  static_assert(KS % 4 == 0 && (16 * NCH) % 256 == 0 && NCH % 8 == 0, "unsupported record width");
  __shared__ int32_t ids[kWidePagesPerBlock];
  __shared__ uint4 tile[2][16 * NCH];
  __shared__ f32x4_t part[2][4][NT][kWave];
  __shared__ uint4 rrec[NCH];

  const int b = blockIdx.z, g = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int n = a.seq_lens[b];
  const int P = (n + kPage - 1) / kPage;
  const bool dense = a.topk >= P;
  const int start = blockIdx.x * ppb;
  if (start >= P) return;
  int end = min(start + ppb, P);
  const int plast = P - 1;
  const bool do_refresh = a.refresh && plast < end;
  if (dense && !do_refresh) return;
  if (a.refresh) end = min(end, plast);
  const int32_t* ptrow = a.page_table + (int64_t)b * a.MP;
  const uint16_t* qrow_b = a.q + ((int64_t)b * a.Hq + (int64_t)g * G) * D;
  const bool SUM = a.head_sum != 0;
  float* srow = a.scores + ((int64_t)b * Hkv + g) * a.MP;

  if (!dense && end > start) stage_i32<kWidePagesPerBlock / 256>(ptrow + start, end - start, ids);
  // this wave's q-/q+ fragments: head 16nt + col, k-chunk kq + 4*(KW*wave + ks)
  uint4 qb[NT][KW];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ks = 0; ks < KW; ++ks) qb[nt][ks] = qq_chunk(qrow_b, nt * 16 + col, G, D, kq + 4 * (KW * wave + ks));
  __syncthreads();

  // partial tiles -> KV-head scores of pages base + 4*kq + wave (lanes col == 0 store)
  auto finish = [&](const f32x4_t (&s)[NT], int buf, int base, int lim) {
    // scaled on the vector ALU before the LDS store (the store never reads an
    // accumulator straight out of the matrix core)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4_t u;
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = s[nt][i] * a.scale;
      part[buf][wave][nt][lane] = u;
    }
    __syncthreads();
    float v = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float x = part[buf][0][nt][lane][wave];
#pragma unroll
      for (int w = 1; w < 4; ++w) x += part[buf][w][nt][lane][wave];
      const bool real = nt * 16 + col < G;
      x = real ? x : (SUM ? 0.f : -__builtin_inff());
      v = nt == 0 ? x : (SUM ? v + x : fmaxf(v, x));
    }
    v = SUM ? group_sum<16>(v) : group_max_any<16>(v);
    const int p = base + 4 * kq + wave;
    if (col == 0 && p < lim) srow[p] = v;
  };

  const uint16_t* summ_g = a.summ + (int64_t)g * 2 * D;
  const int64_t pid_stride = (int64_t)Hkv * 2 * D;
  int buf = 0;
  if (!dense && start < end) {
    const int npg = end - start;
    const int ntile = (npg + 15) / 16;
    // chunk u = c*256 + tid of the tile: page u / NCH, chunk u % NCH
    auto load = [&](int t, uint4 (&r)[CPT]) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int u = c * 256 + threadIdx.x;
        const int p = min(16 * t + u / NCH, npg - 1);
        r[c] = ldnt16(summ_g + (int64_t)ids[p] * pid_stride + 8 * (u % NCH));
      }
    };
    auto stage = [&](int tb, const uint4 (&r)[CPT]) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int u = c * 256 + threadIdx.x;
        const int pg = u / NCH, ch = u % NCH;
        tile[tb][pg * NCH + (ch ^ (pg & 7))] = r[c];
      }
    };
    auto score = [&](int t) {
      const int tb = t & 1;
      f32x4_t s[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KW; ++ks) {
        const int ch = kq + 4 * (KW * wave + ks);
        const uint4 av = tile[tb][col * NCH + (ch ^ (col & 7))];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[nt] = mfma16(av, qb[nt][ks], s[nt]);
      }
      finish(s, buf, start + 16 * t, end);
      buf ^= 1;
    };
    // RD tiles in the register ring: RD - 1 in flight while one is staged and
    // scored (the block is alone on its CU, so deep prefetch keeps HBM busy)
    uint4 r[RD][CPT];
#pragma unroll
    for (int j = 0; j < RD - 1; ++j) load(min(j, ntile - 1), r[j]);
    for (int t = 0; t < ntile; t += RD) {
#pragma unroll
      for (int j = 0; j < RD; ++j) {
        if (j == 0 || t + j < ntile) {
          stage((t + j) & 1, r[j]);
          __syncthreads();
          load(min(t + j + RD - 1, ntile - 1), r[(j + RD - 1) % RD]);
          __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
          score(t + j);
        }
      }
    }
  }

  if (do_refresh) {
    // rebuild the last page's summary from its valid keys, store it, score it
    const int64_t pid = ptrow[plast];
    const int valid = n - plast * kPage;
    const int dc = D / 8;
    uint16_t* rec = a.summ + (pid * Hkv + g) * 2 * D;
    for (int ci = threadIdx.x; ci < NCH; ci += blockDim.x) {
      uint4 mn, mx;
      minmax8(a.k + pid * ps + (int64_t)g * hs + 8 * (ci < dc ? ci : ci - dc), ts, valid, mn, mx);
      const uint4 v = ci < dc ? mn : mx;
      *reinterpret_cast<uint4*>(rec + 8 * ci) = v;
      rrec[ci] = v;
    }
    __syncthreads();
    if (!dense) {
      f32x4_t s[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        s[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KW; ++ks) {
          const uint4 d = col == 0 ? rrec[kq + 4 * (KW * wave + ks)] : make_uint4(0, 0, 0, 0);
          s[nt] = mfma16(d, qb[nt][ks], s[nt]);
        }
      }
      finish(s, buf, plast, plast + 1);  // page slot 0 of the tile is the last page
    }
  }
}

static int pick_ppw(int B, int Hkv, int MP) {
  // about 3072 waves: 768 blocks, the three per CU that the matrix-core
  // kernel's LDS allows, all resident at once (measured: fewer waves leave
  // HBM idle, a second round of blocks costs more than it hides); between 32
  // and kMaxPagesPerWave pages each
  const int64_t pages = (int64_t)B * Hkv * MP;
  int64_t ppw = (pages + 3071) / 3072;
  ppw = (ppw + 31) / 32 * 32;
  if (ppw < 32) ppw = 32;
  if (ppw > kMaxPagesPerWave) ppw = kMaxPagesPerWave;
  return (int)ppw;
}

template <int G, int D>
static hipError_t launch_reg(const Layout& L, const ScoreArgs& a, hipStream_t st) {
  const int ppw = pick_ppw(a.B, L.hkv, a.MP);
  dim3 grid((a.MP + 4 * ppw - 1) / (4 * ppw), L.hkv, a.B);
  if (a.head_sum)
    hipLaunchKernelGGL((quest_score_reg_kernel<G, D, true>), grid, dim3(256), 0, st, a, L.hkv, L.ps, L.hs, L.ts, ppw);
  else
    hipLaunchKernelGGL((quest_score_reg_kernel<G, D, false>), grid, dim3(256), 0, st, a, L.hkv, L.ps, L.hs, L.ts, ppw);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_lds(const Layout& L, const ScoreArgs& a, int G, hipStream_t st) {
  const int ppw = pick_ppw(a.B, L.hkv, a.MP);
  dim3 grid((a.MP + 4 * ppw - 1) / (4 * ppw), L.hkv, a.B);
  const size_t lds = (size_t)2 * G * (D / 8) * sizeof(uint4);
  if (lds > 65536) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)quest_score_lds_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((quest_score_lds_kernel<D>), grid, dim3(256), lds, st, a, G, L.hkv, L.ps, L.hs, L.ts, ppw);
  return hipGetLastError();
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

template <int D, int NT>
static hipError_t launch_wide(const Layout& L, const ScoreArgs& a, int G, hipStream_t st) {
  // whole tiles; at most kWidePagesPerBlock pages per block
  const int64_t pages = (int64_t)a.B * L.hkv * a.MP;
  int64_t ppb = (pages + 255) / 256;  // one block per CU (the LDS tile allows no more)
  ppb = (ppb + 15) / 16 * 16;
  if (ppb < 16) ppb = 16;
  if (ppb > kWidePagesPerBlock) ppb = kWidePagesPerBlock;
  dim3 grid((unsigned)((a.MP + ppb - 1) / ppb), L.hkv, a.B);
  hipLaunchKernelGGL((quest_score_wide_kernel<D, NT, 2>), grid, dim3(256), 0, st, a, G, L.hkv, L.ps, L.hs, L.ts,
                     (int)ppb);
  return hipGetLastError();
}

// Scoring path: the matrix-core kernel unless SE_QUEST_SCORE=valu selects
// the VALU kernels (kept for comparison).
static bool use_valu_scoring() {
  static const bool v = [] {
    const char* e = getenv("SE_QUEST_SCORE");
    return e && strcmp(e, "valu") == 0;
  }();
  return v;
}

hipError_t launch_quest_scores(const Layout& L, const ScoreArgs& a, hipStream_t st) {
  const int G = a.Hq / L.hkv;
  if (a.B == 0 || a.MP == 0) return hipSuccess;
  if (!use_valu_scoring()) {
    if (L.dk == 64) return G <= 16 ? launch_mfma<64, 1>(L, a, G, st) : launch_mfma<64, 2>(L, a, G, st);
    if (L.dk == 128) return G <= 16 ? launch_mfma<128, 1>(L, a, G, st) : launch_mfma<128, 2>(L, a, G, st);
    if (L.dk == 576) return G <= 16 ? launch_wide<576, 1>(L, a, G, st) : launch_wide<576, 2>(L, a, G, st);
    return hipErrorInvalidValue;
  }
#define SE_REG(GG, DD) \
  if (G == GG && L.dk == DD) return launch_reg<GG, DD>(L, a, st);
  SE_REG(1, 64) SE_REG(2, 64) SE_REG(4, 64) SE_REG(8, 64) SE_REG(16, 64)
  SE_REG(1, 128) SE_REG(2, 128) SE_REG(4, 128) SE_REG(8, 128)
#undef SE_REG
  if (L.dk == 64) return launch_lds<64>(L, a, G, st);
  if (L.dk == 128) return launch_lds<128>(L, a, G, st);
  if (L.dk == 576) return launch_lds<576>(L, a, G, st);
  return hipErrorInvalidValue;
}

}  // namespace se
