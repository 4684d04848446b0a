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
  static constexpr int HW = G < (DK <= 128 ? 8 : 4) ? G : (DK <= 128 ? 8 : 4);  // heads per wave
  static constexpr int NHG = G / HW;                                          // head groups
  static constexpr int WPG = NHG >= 4 ? 1 : 4 / NHG;                          // waves per head group
  static constexpr int NW = NHG * WPG;                                        // waves per block
  static constexpr int LPT = DK <= 128 ? 4 : 8;                               // lanes per token, q.k
  static constexpr int TPI = kWave / LPT;                                     // tokens per instruction
  static constexpr int NCK = DK / LPT / 8;                                    // 16-byte chunks per lane
  static constexpr int LPV = DV / 8;                                          // lanes per token, p.v
  static constexpr int TPV = kWave / LPV;                                     // tokens per instruction
  static constexpr int PPS = (DK <= 128 && G <= 16) ? 32 : 16;                // max pages per split
  static_assert(G % HW == 0, "group must split into whole head groups");
  static_assert(DK % (LPT * 8) == 0 && DV % 8 == 0 && LPV <= kWave, "unsupported head dims");
};

template <int G, int DK, int DV, bool VISK>
__global__ __launch_bounds__((DecodeShape<G, DK, DV>::NW * 64)) void decode_kernel(DecodeArgs a, int Hkv, int64_t ps,
                                                                                  int64_t hs, int64_t ts, int pps,
                                                                                  float scale2) {
  using S = DecodeShape<G, DK, DV>;
  constexpr int HW = S::HW, WPG = S::WPG, NW = S::NW, LPT = S::LPT, TPI = S::TPI, NCK = S::NCK;
  constexpr int LPV = S::LPV, TPV = S::TPV, PPS = S::PPS;
  constexpr int RED = WPG > 1 ? NW * HW * DV : 1;

  __shared__ float s_lds[PPS * kPage * G];
  __shared__ float red[RED];
  __shared__ int64_t pid_lds[PPS];
  __shared__ int lp_lds[PPS];
  __shared__ float ml_lds[G][2];

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

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hg = w / WPG, pw = w % WPG;
  const int h0 = hg * HW;
  const uint16_t* kg = a.k + (int64_t)g * hs;

  // ---- phase A: logits ------------------------------------------------------
  {
    const int tok = lane / LPT, j = lane % LPT;
    uint4 qv[HW][NCK];
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
      const uint16_t* qrow = a.q + (head0 + h0 + hh) * DK + 8 * j;
#pragma unroll
      for (int c = 0; c < NCK; ++c) qv[hh][c] = ld16(qrow + 8 * c * LPT);
    }
    for (int i = pw; i < npg; i += WPG) {
      const uint16_t* kb = kg + pid_lds[i] * ps + 8 * j;
      const int pos0 = lp_lds[i] * kPage;
#pragma unroll
      for (int tg = 0; tg < kPage / TPI; ++tg) {
        const int t = tg * TPI + tok;
        uint4 kd[NCK];
#pragma unroll
        for (int c = 0; c < NCK; ++c) kd[c] = ld16(kb + t * ts + 8 * c * LPT);
        const bool valid = pos0 + t < n;
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < NCK; ++c) acc = dot8(qv[hh][c], kd[c], acc);
          acc = group_sum<LPT>(acc) * scale2;
          if (hh % LPT == j) s_lds[(i * kPage + t) * G + h0 + hh] = valid ? acc : -__builtin_inff();
        }
      }
    }
  }
  __syncthreads();

  // ---- phase B: per-head max and exponentials ---------------------------------
  const int T = npg * kPage;
  for (int h = w; h < G; h += NW) {
    float m = -__builtin_inff();
    for (int t = lane; t < T; t += kWave) m = fmaxf(m, s_lds[t * G + h]);
    m = wave_max(m);
    float l = 0.f;
    for (int t = lane; t < T; t += kWave) {
      const float p = __builtin_amdgcn_exp2f(s_lds[t * G + h] - m);
      s_lds[t * G + h] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      ml_lds[h][0] = m;
      ml_lds[h][1] = l;
    }
  }
  __syncthreads();

  // ---- phase C: weighted values ----------------------------------------------
  const int vt = lane / LPV, vc = lane % LPV;
  float acc[HW][8];
#pragma unroll
  for (int hh = 0; hh < HW; ++hh)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[hh][c] = 0.f;
  const uint16_t* vg = (VISK ? a.k : a.v) + (int64_t)g * hs + 8 * vc;
  for (int i = pw; i < npg; i += WPG) {
    const uint16_t* vb = vg + pid_lds[i] * ps;
    const int valid = min(kPage, n - lp_lds[i] * kPage);
#pragma unroll
    for (int tg = 0; tg < kPage / TPV; ++tg) {
      const int t = tg * TPV + vt;
      const uint4 vd = ld16(vb + t * ts);
      float vf[8] = {bf_lo(vd.x), bf_hi(vd.x), bf_lo(vd.y), bf_hi(vd.y),
                     bf_lo(vd.z), bf_hi(vd.z), bf_lo(vd.w), bf_hi(vd.w)};
      if (valid < kPage && t >= valid) {
#pragma unroll
        for (int c = 0; c < 8; ++c) vf[c] = 0.f;  // slots past the sequence may hold anything
      }
      const float* prow = s_lds + (i * kPage + t) * G + h0;
      float p[HW];
#pragma unroll
      for (int hh = 0; hh < HW; ++hh) p[hh] = prow[hh];
#pragma unroll
      for (int hh = 0; hh < HW; ++hh)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[hh][c] = fmaf(p[hh], vf[c], acc[hh][c]);
    }
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
  } else {
    if (vt == 0) {
#pragma unroll
      for (int hh = 0; hh < HW; ++hh)
#pragma unroll
        for (int c = 0; c < 8; ++c) red[((hg * WPG + pw) * HW + hh) * DV + 8 * vc + c] = acc[hh][c];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * DV; idx += blockDim.x) {
      const int h = idx / DV, c = idx % DV;
      const int hgi = h / HW, hh = h % HW;
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < WPG; ++q) s += red[((hgi * WPG + q) * HW + hh) * DV + c];
      a.part_acc[((head0 + h) * nsplit + sbase) * DV + c] = s;
    }
  }
  for (int h = threadIdx.x; h < G; h += blockDim.x) {
    a.part_ml[((head0 + h) * nsplit + sbase) * 2] = ml_lds[h][0];
    a.part_ml[((head0 + h) * nsplit + sbase) * 2 + 1] = ml_lds[h][1];
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
