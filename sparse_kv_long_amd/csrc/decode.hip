// Gathered split-K GQA decode attention over selected 16-token pages, and the
// log-sum-exp merge of the splits, for gfx950.
//
// What is computed (SparseEngine appendix Table 7: logit z between the query
// and a key, normalised weight alpha; the causal history includes the current
// token): for every query head h of KV head g, softmax attention of q_h over
// the valid tokens (t < seq_len) of the pages kept for (request, g) -- all of
// the request's pages in dense mode.
//
// One block per (split, KV head, request).  A split owns up to PPS kept pages.
//   phase A  q.k: LPT lanes share a token row (16-byte loads of LPT adjacent
//            chunks per instruction), q of the wave's HW heads sits in
//            registers, v_dot2 partial sums are combined over the LPT lanes
//            with DPP.  Logits (log2 domain) go to LDS, token-major.
//   phase B  per head: max and sum of 2^(z - max) over the split's tokens.
//   phase C  p.v: each lane owns 8 value channels of one token row, heads'
//            weights are read from LDS, fp32 FMA accumulation; the token
//            groups are then folded together with cross-lane shuffles.
// The split writes (max, sum, unnormalised acc); the merge kernel combines the
// splits of each head: out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
#include "common.h"
#include "se_internal.h"

namespace se {

template <int G, int DK, int DV>
struct DecodeShape {
  static constexpr int HWMAX = DK <= 128 ? 8 : 4;
  static constexpr int HW = G < HWMAX ? G : HWMAX;           // heads per wave
  static constexpr int NHG = G / HW;                          // head groups
  static constexpr int WPG = NHG >= 4 ? 1 : 4 / NHG;          // waves per head group (they split the pages)
  static constexpr int NW = NHG * WPG;                        // waves per block
  static constexpr int LPT = DK <= 128 ? 4 : 8;               // lanes per token, q.k
  static constexpr int TPI = kWave / LPT;                     // tokens per instruction, q.k
  static constexpr int NTG = kPage / TPI;                     // token groups per page, q.k
  static constexpr int NCK = DK / LPT / 8;                    // 16-byte chunks per lane, q.k
  static constexpr int LPV = DV / 8;                          // lanes per token, p.v
  static constexpr int TPV = kWave / LPV;                     // tokens per instruction, p.v
  static constexpr int NTV = kPage / TPV;                     // token groups per page, p.v
  static constexpr int PPS = (DK <= 128 && G <= 16) ? 32 : 16;  // max pages per split
  static constexpr int PPW = (PPS + WPG - 1) / WPG;           // max pages per wave
  static constexpr int LPH = kWave / HW;                      // lanes per head, softmax
  static constexpr bool PREF_A = NTG * NCK * 4 <= 32;         // double-buffer K in registers
  static_assert(G % HW == 0, "group must split into whole head groups");
  static_assert(DK % (LPT * 8) == 0 && DV % 8 == 0 && LPV <= kWave, "unsupported head dims");
};

// Each wave runs q.k -> softmax -> p.v on its own pages with wave-private
// LDS; the only block barriers are after the page-id staging and before the
// final merge of the waves that share a head group.
template <int G, int DK, int DV, bool VISK>
__global__ __launch_bounds__((DecodeShape<G, DK, DV>::NW * 64)) void decode_kernel(DecodeArgs a, int Hkv, int64_t ps,
                                                                                    int64_t hs, int64_t ts, int pps,
                                                                                    float scale2) {
  using S = DecodeShape<G, DK, DV>;
  constexpr int HW = S::HW, WPG = S::WPG, NW = S::NW, LPT = S::LPT, TPI = S::TPI, NTG = S::NTG, NCK = S::NCK;
  constexpr int LPV = S::LPV, TPV = S::TPV, NTV = S::NTV, PPS = S::PPS, PPW = S::PPW, LPH = S::LPH;

  __shared__ float s_lds[NW][PPW * kPage * HW];  // per wave: logits, then weights, token-major
  __shared__ float comb[WPG > 1 ? NW * HW * DV : 1];
  __shared__ float wml[NW][HW][2];
  __shared__ int64_t pid_lds[PPS];
  __shared__ int lp_lds[PPS];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int n = a.seq_lens[b];
  const int P = (n + kPage - 1) / kPage;
  const int32_t* list = nullptr;
  int kk = P;
  if (a.selected) {
    kk = min(a.topk, P);
    list = a.selected + ((int64_t)b * Hkv + g) * a.topk;
  }
  const int p_begin = split * pps;
  const int npg = max(0, min(p_begin + pps, kk) - p_begin);
  const int nsplit = gridDim.x;
  const int64_t head0 = (int64_t)b * a.Hq + (int64_t)g * G;  // first query head of this KV head
  if (npg == 0) {
    // empty split: the merge skips splits whose max is -inf
    for (int h = threadIdx.x; h < G; h += blockDim.x) {
      a.part_ml[((head0 + h) * nsplit + split) * 2] = -__builtin_inff();
      a.part_ml[((head0 + h) * nsplit + split) * 2 + 1] = 0.f;
    }
    return;
  }
  for (int i = threadIdx.x; i < npg; i += blockDim.x) {
    const int lp = list ? list[p_begin + i] : p_begin + i;
    lp_lds[i] = lp;
    pid_lds[i] = a.page_table[(int64_t)b * a.MP + lp];
  }
  __syncthreads();

  // wave index made scalar so that the page loops below branch on scalars
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hg = w / WPG, pw = w % WPG;
  const int h0 = hg * HW;
  const int npw = npg > pw ? (npg - pw + WPG - 1) / WPG : 0;  // pages of this wave: pw + WPG*ii
  float* sw = s_lds[w];

  // ---- phase A: logits (log2 domain) -----------------------------------------
  {
    const int tok = lane / LPT, j = lane % LPT;
    uint4 qv[HW][NCK];
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
      const uint16_t* qrow = a.q + (head0 + h0 + hh) * DK + 8 * j;
#pragma unroll
      for (int c = 0; c < NCK; ++c) qv[hh][c] = ld16(qrow + 8 * c * LPT);
    }
    const uint16_t* kg = a.k + (int64_t)g * hs + 8 * j;
    auto loadk = [&](int ii, uint4 (&kd)[NTG][NCK]) {
      const uint16_t* kb = kg + pid_lds[pw + WPG * ii] * ps;
#pragma unroll
      for (int tg = 0; tg < NTG; ++tg)
#pragma unroll
        for (int c = 0; c < NCK; ++c) kd[tg][c] = ldnt16(kb + (tg * TPI + tok) * ts + 8 * c * LPT);
    };
    auto scorek = [&](int ii, const uint4 (&kd)[NTG][NCK]) {
      const int pos0 = lp_lds[pw + WPG * ii] * kPage;
#pragma unroll
      for (int tg = 0; tg < NTG; ++tg) {
        const int t = tg * TPI + tok;
        const bool valid = pos0 + t < n;
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < NCK; ++c) acc = dot8(qv[hh][c], kd[tg][c], acc);
          acc = group_sum<LPT>(acc) * scale2;
          if (hh % LPT == j) sw[(ii * kPage + t) * HW + hh] = valid ? acc : -__builtin_inff();
        }
      }
    };
    if constexpr (S::PREF_A) {
      // loads are unconditional (index clamped; a clamped load re-reads a
      // cached page) so no branch sits between a prefetch and its use
      uint4 kA[NTG][NCK], kB[NTG][NCK];
      if (npw > 0) {
        loadk(0, kA);
        for (int ii = 0; ii < npw; ii += 2) {
          loadk(min(ii + 1, npw - 1), kB);
          __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
          scorek(ii, kA);
          loadk(min(ii + 2, npw - 1), kA);
          __builtin_amdgcn_sched_barrier(0);
          if (ii + 1 < npw) scorek(ii + 1, kB);
        }
      }
    } else {
      for (int ii = 0; ii < npw; ++ii) {
        uint4 kd[NTG][NCK];
        loadk(ii, kd);
        scorek(ii, kd);
      }
    }
  }

  // ---- value prefetch for the first page, then phase B -------------------------
  const int vt = lane / LPV, vc = lane % LPV;
  const uint16_t* vg = (VISK ? a.k : a.v) + (int64_t)g * hs + 8 * vc;
  auto loadv = [&](int ii, uint4 (&vd)[NTV]) {
    const uint16_t* vb = vg + pid_lds[pw + WPG * ii] * ps;
#pragma unroll
    for (int tg = 0; tg < NTV; ++tg) vd[tg] = ldnt16(vb + (tg * TPV + vt) * ts);
  };
  uint4 vA[NTV], vB[NTV];
  if (npw > 0) loadv(0, vA);  // in flight during the softmax
  __builtin_amdgcn_sched_barrier(0);

  __builtin_amdgcn_wave_barrier();
  {
    const int T = npw * kPage;
    const int hh = lane / LPH, r = lane % LPH;
    float m = -__builtin_inff();
    for (int t = r; t < T; t += LPH) m = fmaxf(m, sw[t * HW + hh]);
    m = group_max_any<LPH>(m);
    float l = 0.f;
    for (int t = r; t < T; t += LPH) {
      const float p = __builtin_amdgcn_exp2f(sw[t * HW + hh] - m);
      sw[t * HW + hh] = p;
      l += p;
    }
    l = group_sum_any<LPH>(l);
    if (r == 0) {
      wml[w][hh][0] = m;
      wml[w][hh][1] = l;
    }
  }
  __builtin_amdgcn_wave_barrier();

  // ---- phase C: weighted values -----------------------------------------------
  float acc[HW][8];
#pragma unroll
  for (int hh = 0; hh < HW; ++hh)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[hh][c] = 0.f;
  auto accum = [&](int ii, const uint4 (&vd)[NTV]) {
    const int valid = min(kPage, n - lp_lds[pw + WPG * ii] * kPage);
#pragma unroll
    for (int tg = 0; tg < NTV; ++tg) {
      const int t = tg * TPV + vt;
      float vf[8] = {bf_lo(vd[tg].x), bf_hi(vd[tg].x), bf_lo(vd[tg].y), bf_hi(vd[tg].y),
                     bf_lo(vd[tg].z), bf_hi(vd[tg].z), bf_lo(vd[tg].w), bf_hi(vd[tg].w)};
      if (valid < kPage && t >= valid) {
#pragma unroll
        for (int c = 0; c < 8; ++c) vf[c] = 0.f;  // slots past the sequence may hold anything
      }
      const float* prow = sw + (ii * kPage + t) * HW;
      float p[HW];
#pragma unroll
      for (int hh = 0; hh < HW; ++hh) p[hh] = prow[hh];
#pragma unroll
      for (int hh = 0; hh < HW; ++hh)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[hh][c] = fmaf(p[hh], vf[c], acc[hh][c]);
    }
  };
  for (int ii = 0; ii < npw; ii += 2) {
    loadv(min(ii + 1, npw - 1), vB);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
    accum(ii, vA);
    loadv(min(ii + 2, npw - 1), vA);
    __builtin_amdgcn_sched_barrier(0);
    if (ii + 1 < npw) accum(ii + 1, vB);
  }
  // fold the TPV token groups of the wave
#pragma unroll
  for (int o = LPV; o < kWave; o <<= 1)
#pragma unroll
    for (int hh = 0; hh < HW; ++hh)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[hh][c] += __shfl_xor(acc[hh][c], o);

  const int64_t sbase = (int64_t)split;
  if constexpr (WPG == 1) {
    if (vt == 0) {
#pragma unroll
      for (int hh = 0; hh < HW; ++hh) {
        float* dst = a.part_acc + ((head0 + h0 + hh) * nsplit + sbase) * DV + 8 * vc;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
      }
    }
    if (lane < HW) {
      a.part_ml[((head0 + h0 + lane) * nsplit + sbase) * 2] = wml[w][lane][0];
      a.part_ml[((head0 + h0 + lane) * nsplit + sbase) * 2 + 1] = wml[w][lane][1];
    }
  } else {
    if (vt == 0) {
#pragma unroll
      for (int hh = 0; hh < HW; ++hh)
#pragma unroll
        for (int c = 0; c < 8; ++c) comb[(w * HW + hh) * DV + 8 * vc + c] = acc[hh][c];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * (DV + 2); idx += blockDim.x) {
      const int h = idx / (DV + 2), c = idx % (DV + 2);
      const int hgi = h / HW, hh = h % HW;
      float M = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < WPG; ++q) M = fmaxf(M, wml[hgi * WPG + q][hh][0]);
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < WPG; ++q) {
        const float mq = wml[hgi * WPG + q][hh][0];
        const float f = mq == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mq - M);
        const float v = c < DV ? comb[((hgi * WPG + q) * HW + hh) * DV + c] : wml[hgi * WPG + q][hh][1];
        s += f * v;
      }
      if (c < DV)
        a.part_acc[((head0 + h) * nsplit + sbase) * DV + c] = s;
      else if (c == DV)
        a.part_ml[((head0 + h) * nsplit + sbase) * 2] = M;
      else
        a.part_ml[((head0 + h) * nsplit + sbase) * 2 + 1] = s;
    }
  }
}

// One block per (request, query head).
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part_acc,
                                                    const float* __restrict__ part_ml, float* __restrict__ out,
                                                    int nsplit, int DV) {
  const int64_t bh = blockIdx.x;
  const float* ml = part_ml + bh * nsplit * 2;
  float M = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float den = 0.f;
  for (int s = 0; s < nsplit; ++s)
    if (ml[2 * s] != -__builtin_inff()) den += __builtin_amdgcn_exp2f(ml[2 * s] - M) * ml[2 * s + 1];
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int c = threadIdx.x; c < DV; c += blockDim.x) {
    float num = 0.f;
    for (int s = 0; s < nsplit; ++s)
      if (ml[2 * s] != -__builtin_inff())
        num += __builtin_amdgcn_exp2f(ml[2 * s] - M) * part_acc[(bh * nsplit + s) * DV + c];
    out[bh * DV + c] = num * inv;
  }
}

static int max_pps(const Layout& L, int G) { return (L.dk <= 128 && G <= 16) ? 32 : 16; }

int decode_splits(const Layout& L, int B, int Hq, int MP, int topk, bool dense, int requested) {
  // pages attended per (request, KV head) at most
  const int kmax = (dense || topk >= MP) ? MP : topk;
  if (kmax <= 0) return 1;
  const int units = B * L.hkv;
  const int mp = max_pps(L, Hq / L.hkv);
  const int smin = (kmax + mp - 1) / mp;
  int s = requested > 0 ? requested : (1024 + units - 1) / units;
  if (s < smin) s = smin;
  if (s > kmax) s = kmax;
  const int pps = (kmax + s - 1) / s;
  return (kmax + pps - 1) / pps;
}

size_t decode_partials_bytes(const Layout& L, int B, int Hq, int splits) {
  return (size_t)B * Hq * splits * (L.dv + 2) * sizeof(float);
}

template <int G, int DK, int DV, bool VISK>
static hipError_t launch_g(const Layout& L, const DecodeArgs& a, int pps, hipStream_t st) {
  using S = DecodeShape<G, DK, DV>;
  const float scale2 = a.scale * kLog2e;
  dim3 grid(a.splits, L.hkv, a.B);
  hipLaunchKernelGGL((decode_kernel<G, DK, DV, VISK>), grid, dim3(S::NW * 64), 0, st, a, L.hkv, L.ps, L.hs, L.ts,
                     pps, scale2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(a.B * a.Hq), dim3(128), 0, st, a.part_acc, a.part_ml, a.out, a.splits, DV);
  return hipGetLastError();
}

template <int DK, int DV, bool VISK>
static hipError_t launch_d(const Layout& L, const DecodeArgs& a, int G, int pps, hipStream_t st) {
  switch (G) {
    case 1: return launch_g<1, DK, DV, VISK>(L, a, pps, st);
    case 2: return launch_g<2, DK, DV, VISK>(L, a, pps, st);
    case 4: return launch_g<4, DK, DV, VISK>(L, a, pps, st);
    case 8: return launch_g<8, DK, DV, VISK>(L, a, pps, st);
    case 16: return launch_g<16, DK, DV, VISK>(L, a, pps, st);
    case 32: return launch_g<32, DK, DV, VISK>(L, a, pps, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const Layout& L, const DecodeArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / L.hkv;
  const int kmax = a.selected ? (a.topk < a.MP ? a.topk : a.MP) : a.MP;
  const int pps = (kmax + a.splits - 1) / a.splits;
  if (pps > max_pps(L, G)) return hipErrorInvalidValue;
  if (L.dk == 64 && L.dv == 64 && !L.visk) return launch_d<64, 64, false>(L, a, G, pps, st);
  if (L.dk == 128 && L.dv == 128 && !L.visk) return launch_d<128, 128, false>(L, a, G, pps, st);
  if (L.dk == 576 && L.dv == 512 && L.visk) return launch_d<576, 512, true>(L, a, G, pps, st);
  return hipErrorInvalidValue;
}

}  // namespace se
