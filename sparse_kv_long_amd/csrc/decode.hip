// Gathered split-K GQA decode attention over selected 16-token pages, and the
// log-sum-exp merge of the splits, for gfx950.
//
// What is computed (SparseEngine appendix Table 7: logit z between the query
// and a key, normalised weight alpha; the causal history includes the current
// token): for every query head h of KV head g, softmax attention of q_h over
// the valid tokens (t < seq_len) of the pages kept for (request, g) -- all of
// the request's pages in dense mode.
//
// Three kernels compute it, one block per (split, KV head, request), a split
// owning up to PPS kept pages: the matrix-core kernel for head dimension 128
// with up to 16 query heads per KV head (decode_mfma_kernel), the one for the
// 576/512 latent layout (decode_mla_kernel), and a vector-ALU kernel for the
// other shapes, or for every shape when the caller asks for it
// (decode_kernel).  Each split writes (max, sum, unnormalised acc) -- or,
// when it is the request's only split, the matrix-core GQA kernel writes the
// output itself -- and the merge kernel combines the splits of each head:
// out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
#include "common.h"
#include "se_internal.h"

namespace se {

// Online softmax with a lazily moved reference max (log2 units): the matrix-
// core decodes rescale their accumulators only when a head's running max
// grows by more than this, so every weight stays below 2^kLazyRescale (no
// overflow in fp32, and the bf16 hi + lo split keeps its relative accuracy)
// and the rescale, which touches every accumulator, runs on few pages.
constexpr float kLazyRescale = 8.f;

template <int G, int DK, int DV>
struct DecodeShape {
  static constexpr int HWMAX = DK <= 128 ? 8 : 4;
  static constexpr int HW = G < HWMAX ? G : HWMAX;           // heads per wave
  static constexpr int NHG = G / HW;                          // head groups
  static constexpr int WPG = NHG >= 4 ? 1 : 4 / NHG;          // waves per head group (they split the pages)
  static constexpr int NW = NHG * WPG;                        // waves per block
  static constexpr int LPT = 8;                               // lanes per token, q.k
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

// Vector-ALU decode.  Each wave runs q.k -> softmax -> p.v on its own pages
// with wave-private LDS; the only block barriers are after the page-id
// staging and before the final merge of the waves that share a head group.
//   phase A  q.k: LPT lanes share a token row (16-byte loads of LPT adjacent
//            chunks per instruction), q of the wave's HW heads sits in
//            registers, v_dot2 partial sums are combined over the LPT lanes
//            with DPP.  Logits (log2 domain) go to LDS, token-major.
//   phase B  per head: max and sum of 2^(z - max) over the wave's tokens.
//   phase C  p.v: each lane owns 8 value channels of one token row, heads'
//            weights are read from LDS, fp32 FMA accumulation; the token
//            groups are then folded together with cross-lane shuffles.
template <int G, int DK, int DV, bool VISK>
__global__ __launch_bounds__((DecodeShape<G, DK, DV>::NW * 64))
__attribute__((amdgpu_waves_per_eu(DK > 128 ? 2 : G == 16 ? 3 : 4))) void decode_kernel(DecodeArgs a, int Hkv,
                                                                                        int64_t ps, int64_t hs,
                                                                                        int64_t ts, int pps,
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

// ---------------------------------------------------------------------------
// Matrix-core decode for Dk = Dv = 128 and G <= 16 (one 16-row head tile).
//
//   q.k   S[t][h] = sum_c K[t][c] q[h][c]: v_mfma_f32_16x16x32_bf16 with the
//         page's 16 tokens as rows, 4 k-steps of 32 channels; lane l loads
//         token l%16, channels 8*(l/16) + 32*ks (16 bytes).  Exact bf16
//         products, fp32 accumulation.
//   p.v   O[h][c] = sum_t P[h][t] V[t][c], one page (16 tokens) per
//         v_mfma_f32_16x16x32_bf16: value rows are loaded whole (lane l:
//         tokens 4e + l/16, channels 8*(l%16)..+7), so a lane owns 8 channels
//         of 4 tokens; N-tile nt takes channels {8n + nt}, which makes every
//         B-fragment a 2 x v_perm_b32 repack of the lane's own registers.
//         P enters as a hi + lo pair of bf16 (P = hi + lo to ~2^-16): the
//         32-wide k dimension holds the hi parts of the lane's 4 tokens, then
//         their lo parts, against the same 4 value rows repeated, so the
//         weights keep near-fp32 precision at one MFMA per tile.
// Softmax, masking, the split partials and the merge are as in the VALU
// kernel.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ uint32_t dword(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int G>
struct MfmaDecodeShape {
  static constexpr int PPS = G <= 8 ? 256 : 128;  // max pages per split (ids staged in LDS)
};

// One block of NW waves per (split, KV head, request); wave w streams pages
// w, w+NW, ... of the split with an online softmax, keeping the K and V
// loads of the next two pages in flight.  Lane l = 16*kq + col.  FINAL (one
// split): the block normalises and writes the output itself, no merge.
//   q.k   A = K (lane: token col, channels 8kq + 32ks), B = q (head col);
//         output lane (col, kq): tokens 4kq + i of the page, head col.
//   p.v   A = P (lane: head col, k 8kq + j = hi (j < 4) / lo (j >= 4) of
//         token 4kq + j%4), B = V (lane: channels 8col + nt, the same tokens)
//         -- the weights stay in the lanes that computed them, and the value
//         rows are loaded whole (16 lanes per 256-byte row) and repacked
//         in-lane with v_perm_b32.
// Two waves per SIMD, declared as such: the accumulators then live in
// ordinary vector registers, with no copies into and out of the
// accumulation registers (measured 0.3-0.8 us faster at 128K and 32K).
template <int G, int NW, bool FINAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void
decode_mfma_kernel(DecodeArgs a, int Hkv, int64_t ps, int64_t hs, int64_t ts, int pps, float scale2) {
  constexpr int D = 128, PPS = MfmaDecodeShape<G>::PPS;
  static_assert(G <= 16, "one 16-row head tile");
  __shared__ float head_ml[16][2];  // FINAL: per head, the max and the weight sum over the waves
  __shared__ float comb[NW * G * D];
  __shared__ float wml[NW][G][2];
  __shared__ float alpha_lds[NW][16];
  __shared__ uint4 kstage[NW][kPage * 16];  // per wave: 16 tokens x 16 chunks of 8 channels, swizzled
  __shared__ int64_t pid_lds[PPS];
  __shared__ int vld_lds[PPS];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nsplit = gridDim.x;
  const int64_t head0 = (int64_t)b * a.Hq + (int64_t)g * G;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  // The request's length, q and the split's page ids are requested together,
  // before any of them is used: the ids are read up to the split's nominal
  // size within their row (entries past the request's pages are staged but
  // never used), so the first page loads wait for one memory round trip
  // instead of three dependent ones.
  const int n = a.seq_lens[b];
  uint4 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = ld16(a.q + (head0 + min(col, G - 1)) * D + 8 * kq + 32 * ks);  // unconditional: loads issue together
  const int32_t* list = nullptr;
  const int32_t* plist = nullptr;
  if (a.selected) {
    list = a.selected + ((int64_t)b * Hkv + g) * a.topk;
    if (a.selected_phys) plist = a.selected_phys + ((int64_t)b * Hkv + g) * a.topk;
  }
  const int p_begin = split * pps;
  const int rowlen = a.selected ? a.topk : a.MP;
  for (int i = threadIdx.x; i < pps; i += blockDim.x) {
    const int idx = min(p_begin + i, rowlen - 1);
    const int lp = list ? list[idx] : idx;
    pid_lds[i] = plist ? plist[idx] : a.page_table[(int64_t)b * a.MP + min(max(lp, 0), a.MP - 1)];
    vld_lds[i] = lp;  // turned into a token count below, by the same thread
  }
  const int P = (n + kPage - 1) / kPage;
  const int kk = a.selected ? min(a.topk, P) : P;
  const int npg = max(0, min(p_begin + pps, kk) - p_begin);
  if (npg == 0) {
    if (FINAL) {  // an empty request: a zero output row
      for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) a.out[head0 * D + idx] = 0.f;
      return;
    }
    for (int h = threadIdx.x; h < G; h += blockDim.x) {
      a.part_ml[((head0 + h) * nsplit + split) * 2] = -__builtin_inff();
      a.part_ml[((head0 + h) * nsplit + split) * 2 + 1] = 0.f;
    }
    return;
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    if (col >= G) qf[ks] = make_uint4(0, 0, 0, 0);
  for (int i = threadIdx.x; i < npg; i += blockDim.x) vld_lds[i] = min(kPage, n - vld_lds[i] * kPage);
  __syncthreads();

  const int npw = npg > w ? (npg - w + NW - 1) / NW : 0;  // pages of this wave: w + NW*ii
  // K and V rows are both loaded whole (lane: rows 4kq + e, channels 8col..+7);
  // K is restaged through this wave's LDS tile into the q.k A layout
  uint4* st = kstage[w];


  struct PageRegs {
    uint4 k[4], v[4];
  };
  // the page base is wave-uniform (scalar registers); each lane adds the same
  // 32-bit byte offsets for K and V rows
  uint32_t roff[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) roff[e] = (uint32_t)(2 * (8 * col + (4 * kq + e) * ts));
  const uint16_t* kh = a.k + (int64_t)g * hs;
  const uint16_t* vh = a.v + (int64_t)g * hs;
  // past the wave's last page the ring's loads go through empty resources:
  // they return zeros and read nothing (a repeat of the last page would be
  // re-fetched: the page loads are non-temporal)
  auto load = [&](int ii, PageRegs& r) {
    const int64_t pid = pid_lds[w + NW * min(ii, npw - 1)];
    const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane((int)pid) * ps;
    const int span = ii < npw ? 0x7fffffff : 0;
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kh + off, span), rv = buf_rsrc(vh + off, span);
#pragma unroll
    for (int e = 0; e < 4; ++e) r.k[e] = ldbuf_nt16(rk, roff[e]);
#pragma unroll
    for (int e = 0; e < 4; ++e) r.v[e] = ldbuf_nt16(rv, roff[e]);
  };

  float m_run = -__builtin_inff();  // running max of head col (log2 domain)
  float l_run = 0.f;                // sum of 2^(z - m_run) over this lane's tokens
  f32x4_t acc[8];                   // rows: heads 4kq + i; columns: channels 8col + nt
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto page = [&](int ii, PageRegs& r) {
    const int valid = vld_lds[w + NW * ii];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * kq + e;
      st[t * 16 + (col ^ (t & 7))] = r.k[e];
    }
    __builtin_amdgcn_wave_barrier();  // lanes read what other lanes wrote
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) s = mfma16(st[col * 16 + ((4 * ks + kq) ^ (col & 7))], qf[ks], s);
    __builtin_amdgcn_wave_barrier();  // the next page's restaging waits for these reads
    float z[4];
    float pm = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = (col < G && 4 * kq + i < valid) ? s[i] * scale2 : -__builtin_inff();
      pm = fmaxf(pm, z[i]);
    }
    pm = rows_max(pm);
    // lazy rescaling: a head's reference max moves only when the page max
    // passes it by more than kLazyRescale, so most pages skip the rescale
    const bool grow = pm > m_run + kLazyRescale;
    if (__any(grow)) {
      const float alpha = !grow ? 1.f : m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - pm);
      l_run *= alpha;
      m_run = grow ? pm : m_run;
      // rescale the accumulators (rows are heads 4kq + i)
      if (kq == 0) alpha_lds[w][col] = alpha;
      __builtin_amdgcn_wave_barrier();
      const float4 al = *reinterpret_cast<const float4*>(&alpha_lds[w][4 * kq]);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        acc[nt][0] *= al.x;
        acc[nt][1] *= al.y;
        acc[nt][2] *= al.z;
        acc[nt][3] *= al.w;
      }
      __builtin_amdgcn_wave_barrier();
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(z[i] - m_run);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    // weights as hi + lo bf16 pairs, elements e = tokens 4kq + e
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t h0 = __float_as_uint(p[2 * d]) & 0xffff0000u, h1 = __float_as_uint(p[2 * d + 1]) & 0xffff0000u;
      const uint32_t l0 = __float_as_uint(p[2 * d] - __uint_as_float(h0));
      const uint32_t l1 = __float_as_uint(p[2 * d + 1] - __uint_as_float(h1));
      hi[d] = (h0 >> 16) | h1;
      lo[d] = (l0 >> 16) | (l1 & 0xffff0000u);
    }
    // k = 8kq + j: j < 4 the hi parts of tokens 4kq + j, j >= 4 the lo parts of the same tokens
    const uint4 pa = make_uint4(hi[0], hi[1], lo[0], lo[1]);
    if (valid < kPage) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * kq + e >= valid) r.v[e] = make_uint4(0, 0, 0, 0);  // slots past the sequence may hold anything
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const uint32_t sel = (nt & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t f0 = __builtin_amdgcn_perm(dword(r.v[1], nt >> 1), dword(r.v[0], nt >> 1), sel);
      const uint32_t f1 = __builtin_amdgcn_perm(dword(r.v[3], nt >> 1), dword(r.v[2], nt >> 1), sel);
      acc[nt] = mfma16(pa, make_uint4(f0, f1, f0, f1), acc[nt]);
    }
  };

  if (npw > 0) {
    PageRegs r0, r1, r2;
    load(0, r0);
    load(1, r1);
    for (int ii = 0; ii < npw; ii += 3) {
      load(ii + 2, r2);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetches ahead of the compute
      page(ii, r0);
      load(ii + 3, r0);
      __builtin_amdgcn_sched_barrier(0);
      if (ii + 1 < npw) page(ii + 1, r1);
      load(ii + 4, r1);
      __builtin_amdgcn_sched_barrier(0);
      if (ii + 2 < npw) page(ii + 2, r2);
    }
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- merge the block's waves and write the split partial ------------------------
  if (kq == 0 && col < G) {
    wml[w][col][0] = m_run;
    wml[w][col][1] = l_run;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * kq + i;
    if (h < G) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) comb[(w * G + h) * D + 8 * col + nt] = acc[nt][i];
    }
  }
  __syncthreads();
  if (FINAL) {
    if (threadIdx.x < G) {
      const int h = threadIdx.x;
      float M = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < NW; ++q) M = fmaxf(M, wml[q][h][0]);
      float L = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const float mq = wml[q][h][0];
        L += mq == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mq - M) * wml[q][h][1];
      }
      head_ml[h][0] = M;
      head_ml[h][1] = L > 0.f ? 1.f / L : 0.f;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
      const int h = idx / D, c = idx % D;
      const float M = head_ml[h][0];
      float sacc = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const float mq = wml[q][h][0];
        sacc += mq == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mq - M) * comb[(q * G + h) * D + c];
      }
      a.out[(head0 + h) * D + c] = sacc * head_ml[h][1];
    }
    return;
  }
  const int64_t sbase = (int64_t)split;
  for (int idx = threadIdx.x; idx < G * (D + 2); idx += blockDim.x) {
    const int h = idx / (D + 2), c = idx % (D + 2);
    float M = -__builtin_inff();
#pragma unroll
    for (int q = 0; q < NW; ++q) M = fmaxf(M, wml[q][h][0]);
    float sacc = 0.f;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      const float mq = wml[q][h][0];
      if (mq == -__builtin_inff()) continue;  // a wave without pages
      const float v = c < D ? comb[(q * G + h) * D + c] : wml[q][h][1];
      sacc += __builtin_amdgcn_exp2f(mq - M) * v;
    }
    if (c < D)
      a.part_acc[((head0 + h) * nsplit + sbase) * D + c] = sacc;
    else if (c == D)
      a.part_ml[((head0 + h) * nsplit + sbase) * 2] = M;
    else
      a.part_ml[((head0 + h) * nsplit + sbase) * 2 + 1] = sacc;
  }
}

// ---------------------------------------------------------------------------
// Matrix-core decode for the MLA layout: one 576-channel key row per token
// (latent 512 + rope 64), the value is the first 512 channels of the same
// row, and up to 32 query heads share it.
//
// One block of 4 waves per (split, block of 16 query heads, KV head,
// request); all four waves walk the same pages.  Wave w owns value channels
// [128w, 128w + 128): it loads those 16 x 128 of each page once (lane: rows
// 4kq + e, channels 8col..+7), uses them as the p.v operand, and, restaged
// through LDS in A-fragment order, for its share of q.k (latent channels
// 128w.., plus rope channels 512 + 16w..).  The four partial logit tiles are
// summed through LDS in a fixed order, so every wave holds the same logits,
// the same running max / sum and the same weights; no merge across waves is
// needed at the end.  One block barrier per pair of pages.  With 16 heads per
// block the kernel fits two waves per SIMD (two blocks per CU); the 32-head
// case runs two head blocks over the same pages, whose second reads of a page
// are served by the caches.
// ---------------------------------------------------------------------------
constexpr int kMlaPagesPerSplit = 512;
constexpr int kMlaTargetBlocks = 512;  // two resident blocks per CU
constexpr int kMlaHeadsPerBlock = 16;
// With an even split count the splits form two halves, the first dispatched
// first: its blocks are the older of the two on each CU and win its issue
// arbitration (clock stamps: their page loops took 15.7 us against 19.4 us),
// so the first half's splits hold about 15% more pages (MLA ragged batch:
// 18 and 14 of 256; decode + merge 35.1 against 35.9 us, 35.3 at 30%)
constexpr int kMlaSplitTilt = 150;  // first-half splits longer by this / 1024

template <int NHT, int RD, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void decode_mla_kernel(DecodeArgs a, int Hkv, int64_t ps, int64_t hs, int64_t ts, int pps, int pps1, float scale2,
                       int nhb) {
  constexpr int DK = 576, DV = 512, NW = 4, PPS = kMlaPagesPerSplit;
  __shared__ uint4 stage[NW][2][kPage * 16];      // per wave and page of the pair: 16 tokens x 16 chunks, swizzled
  __shared__ f32x4_t sbuf[2][NW][2 * NHT][kWave];  // partial logits (head tile, page), double-buffered over pairs
  __shared__ float alpha_lds[NW][NHT * 16];
  __shared__ int64_t pid_lds[PPS];
  __shared__ int vld_lds[PPS];

  // grid x: splits of one half x head blocks (16 * NHT query heads each);
  // z: halves x requests.  The first half's splits (dispatched first) hold
  // pps pages each, the second half's pps1.
  const int halves = gridDim.z / a.B, nsh = gridDim.x / nhb, nsplit = nsh * halves;
  const int half = blockIdx.z / a.B, b = blockIdx.z % a.B, g = blockIdx.y;
  const int split = half * nsh + blockIdx.x % nsh, hblk = blockIdx.x / nsh;
  const int my_pps = half == 0 ? pps : pps1;
  const int Gall = a.Hq / Hkv;
  const int G = min(16 * NHT, Gall - 16 * NHT * hblk);  // query heads of this block
  const int64_t head0 = (int64_t)b * a.Hq + (int64_t)g * Gall + 16 * NHT * hblk;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  // The request's length, q and the split's page ids are requested together,
  // before any of them is used (the ids up to the split's nominal size within
  // their row; entries past the request's pages are staged but never used).
  const int n = a.seq_lens[b];
  // q fragments: head 16ht + col; latent channels 128w + 32ks + 8kq, rope 512 + 16w + 4kq
  uint4 qf[NHT][4];
  uint2 qr[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = 16 * ht + col;
    const uint16_t* qh = a.q + (head0 + min(h, G - 1)) * DK;  // unconditional: the loads issue together
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ht][ks] = ld16(qh + 128 * w + 32 * ks + 8 * kq);
    qr[ht] = *reinterpret_cast<const uint2*>(qh + 512 + 16 * w + 4 * kq);
  }
  const int32_t* list = nullptr;
  const int32_t* plist = nullptr;
  if (a.selected) {
    list = a.selected + ((int64_t)b * Hkv + g) * a.topk;
    if (a.selected_phys) plist = a.selected_phys + ((int64_t)b * Hkv + g) * a.topk;
  }
  const int p_begin = half == 0 ? split * pps : nsh * pps + (split - nsh) * pps1;
  const int rowlen = a.selected ? a.topk : a.MP;
  for (int i = threadIdx.x; i < my_pps; i += blockDim.x) {
    const int idx = min(p_begin + i, rowlen - 1);
    const int lp = list ? list[idx] : idx;
    pid_lds[i] = plist ? plist[idx] : a.page_table[(int64_t)b * a.MP + min(max(lp, 0), a.MP - 1)];
    vld_lds[i] = lp;  // turned into a token count below, by the same thread
  }
  const int P = (n + kPage - 1) / kPage;
  const int kk = a.selected ? min(a.topk, P) : P;
  const int npg = max(0, min(p_begin + my_pps, kk) - p_begin);
  if (npg == 0) {
    for (int h = threadIdx.x; h < G; h += blockDim.x) {
      a.part_ml[((head0 + h) * nsplit + split) * 2] = -__builtin_inff();
      a.part_ml[((head0 + h) * nsplit + split) * 2 + 1] = 0.f;
    }
    return;
  }
  for (int i = threadIdx.x; i < npg; i += blockDim.x) vld_lds[i] = min(kPage, n - vld_lds[i] * kPage);
  const uint16_t* kb = a.k + (int64_t)g * hs;
  const uint16_t* vrow = kb + 128 * w + 8 * col + (4 * kq) * ts;  // + e * ts: value rows 4kq + e
  const uint16_t* rrow = kb + col * ts + 512 + 16 * w + 4 * kq;   // rope: token col, 4 channels
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    if (16 * ht + col >= G) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[ht][ks] = make_uint4(0, 0, 0, 0);
      qr[ht] = make_uint2(0, 0);
    }
  }

  struct PageRegs {
    uint4 v[4];
    uint2 r;
  };
  // byte offsets inside a page (vrow / rrow above, relative to kb); past the
  // block's last page the ring's loads go through an empty resource and read
  // nothing
  uint32_t voff[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) voff[e] = (uint32_t)(2 * ((vrow - kb) + e * ts));
  const uint32_t roff = (uint32_t)(2 * (rrow - kb));
  auto load = [&](int ii, PageRegs& R) {
    const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane((int)pid_lds[min(ii, npg - 1)]) * ps;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(kb + off, ii < npg ? 0x7fffffff : 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) R.v[e] = ldbuf_nt16(rs, voff[e]);
    R.r = ldbuf8(rs, roff);
  };

  float m_run[NHT], l_run[NHT];
  f32x4_t acc[NHT][8];  // rows: heads 16ht + 4kq + i; columns: channels 128w + 8col + nt
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    m_run[ht] = -__builtin_inff();
    l_run[ht] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[ht][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // Pages are consumed in pairs: the softmax chain (row max, exponentials,
  // weight split) is a run of dependent steps whose latency, with one wave
  // per SIMD, nothing else hides; over two pages at once every step has twice
  // the independent work, and the block barrier is paid once per pair.
  auto restage = [&](const PageRegs& R, uint4* st) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * kq + e;
      st[t * 16 + (col ^ (t & 7))] = R.v[e];
    }
  };
  // this wave's share of the logits: rope (k = 8kq + j, channels 512 + 16w +
  // 4kq + j for j < 4, zero above), then the latent slice restaged in st
  auto qk = [&](const PageRegs& R, const uint4* st, f32x4_t (&s)[NHT]) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
      s[ht] = mfma16(make_uint4(R.r.x, R.r.y, 0u, 0u), make_uint4(qr[ht].x, qr[ht].y, 0u, 0u),
                     f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 A = st[col * 16 + ((4 * ks + kq) ^ (col & 7))];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) s[ht] = mfma16(A, qf[ht][ks], s[ht]);
    }
  };
  // value fragments: {channel 8col + nt of tokens 4kq + 0, 1} and {.. 2, 3};
  // rows past the sequence are zeroed (those slots may hold anything)
  auto vfrag = [&](PageRegs& R, int valid, uint32_t (&vfr)[8][2]) {
    if (valid < kPage) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * kq + e >= valid) R.v[e] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const uint32_t sel = (nt & 1) ? 0x07060302u : 0x05040100u;
      vfr[nt][0] = __builtin_amdgcn_perm(dword(R.v[1], nt >> 1), dword(R.v[0], nt >> 1), sel);
      vfr[nt][1] = __builtin_amdgcn_perm(dword(R.v[3], nt >> 1), dword(R.v[2], nt >> 1), sel);
    }
  };
  // weights as hi + lo bf16 pairs along k: k = 8kq + j, hi (j < 4) and lo (j >= 4) of tokens 4kq + j
  auto split_hi_lo = [](const float* p) -> uint4 {
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t h0 = __float_as_uint(p[2 * d]) & 0xffff0000u, h1 = __float_as_uint(p[2 * d + 1]) & 0xffff0000u;
      const uint32_t l0 = __float_as_uint(p[2 * d] - __uint_as_float(h0));
      const uint32_t l1 = __float_as_uint(p[2 * d + 1] - __uint_as_float(h1));
      hi[d] = (h0 >> 16) | h1;
      lo[d] = (l0 >> 16) | (l1 & 0xffff0000u);
    }
    return make_uint4(hi[0], hi[1], lo[0], lo[1]);
  };

  // pages ii and ii + 1 (the second absent, and all its weights zero, when ii + 1 == npg)
  auto pair = [&](int ii, PageRegs& RA, PageRegs& RB) {
    const int vA = vld_lds[ii];
    const int vB = ii + 1 < npg ? vld_lds[ii + 1] : 0;
    const int buf = (ii >> 1) & 1;
    restage(RA, stage[w][0]);
    restage(RB, stage[w][1]);
    __builtin_amdgcn_wave_barrier();  // lanes read what other lanes wrote
    f32x4_t sA[NHT], sB[NHT];
    qk(RA, stage[w][0], sA);
    qk(RB, stage[w][1], sB);
    __builtin_amdgcn_wave_barrier();  // the next pair's restaging waits for these reads
    // sum the four waves' channel shares (scaled to the log2 domain) in a fixed order
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f32x4_t u, v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u[i] = sA[ht][i] * scale2;
        v[i] = sB[ht][i] * scale2;
      }
      sbuf[buf][w][2 * ht][lane] = u;
      sbuf[buf][w][2 * ht + 1][lane] = v;
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f32x4_t t = sbuf[buf][0][2 * ht][lane], t2 = sbuf[buf][0][2 * ht + 1][lane];
#pragma unroll
      for (int q = 1; q < NW; ++q) {
        const f32x4_t u = sbuf[buf][q][2 * ht][lane], v = sbuf[buf][q][2 * ht + 1][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          t[i] += u[i];
          t2[i] += v[i];
        }
      }
      sA[ht] = t;
      sB[ht] = t2;
    }
    uint32_t vfA[8][2], vfB[8][2];
    vfrag(RA, vA, vfA);
    vfrag(RB, vB, vfB);
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const bool hv = 16 * ht + col < G;
      float z[8];
      float pm = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = (hv && 4 * kq + i < vA) ? sA[ht][i] : -__builtin_inff();
        z[4 + i] = (hv && 4 * kq + i < vB) ? sB[ht][i] : -__builtin_inff();
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) pm = fmaxf(pm, z[i]);
      pm = rows_max(pm);
      // lazy rescaling, as in the GQA kernel
      const bool grow = pm > m_run[ht] + kLazyRescale;
      if (__any(grow)) {
        const float alpha =
            !grow ? 1.f : m_run[ht] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run[ht] - pm);
        l_run[ht] *= alpha;
        m_run[ht] = grow ? pm : m_run[ht];
        if (kq == 0) alpha_lds[w][16 * ht + col] = alpha;
        __builtin_amdgcn_wave_barrier();
        const float4 al = *reinterpret_cast<const float4*>(&alpha_lds[w][16 * ht + 4 * kq]);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          acc[ht][nt][0] *= al.x;
          acc[ht][nt][1] *= al.y;
          acc[ht][nt][2] *= al.z;
          acc[ht][nt][3] *= al.w;
        }
        __builtin_amdgcn_wave_barrier();
      }
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(z[i] - m_run[ht]);
      l_run[ht] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      const uint4 paA = split_hi_lo(p), paB = split_hi_lo(p + 4);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        acc[ht][nt] = mfma16(paA, make_uint4(vfA[nt][0], vfA[nt][1], vfA[nt][0], vfA[nt][1]), acc[ht][nt]);
        acc[ht][nt] = mfma16(paB, make_uint4(vfB[nt][0], vfB[nt][1], vfB[nt][0], vfB[nt][1]), acc[ht][nt]);
      }
    }
  };

  {
    // RD pages in the register ring, consumed two at a time (RD - 2 in
    // flight while a pair is processed): the block is alone on its CU, so
    // deep prefetch is what keeps HBM busy
    static_assert(RD % 2 == 0 && RD >= 4, "the ring holds whole pairs");
    PageRegs r[RD];
#pragma unroll
    for (int j = 0; j < RD - 2; ++j) {
      load(j, r[j]);
      __builtin_amdgcn_sched_barrier(0);  // issue order = use order, so each wait covers one page
    }
    for (int ii = 0; ii < npg; ii += RD) {
#pragma unroll
      for (int j = 0; j < RD; j += 2) {
        load(ii + j + RD - 2, r[(j + RD - 2) % RD]);
        load(ii + j + RD - 1, r[(j + RD - 1) % RD]);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetches ahead of the compute
        if (j == 0 || ii + j < npg) pair(ii + j, r[j], r[j + 1]);
      }
    }
  }

  // every wave holds the same (m, l); each writes its 128 channels of the split partial
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    float l = l_run[ht];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int hb = 16 * ht;
    if (w == 0 && kq == 0 && hb + col < G) {
      a.part_ml[((head0 + hb + col) * nsplit + split) * 2] = m_run[ht];
      a.part_ml[((head0 + hb + col) * nsplit + split) * 2 + 1] = l;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hb + 4 * kq + i;
      if (h < G) {
        float* dst = a.part_acc + ((head0 + h) * nsplit + split) * DV + 128 * w + 8 * col;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[ht][0][i], acc[ht][1][i], acc[ht][2][i], acc[ht][3][i]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[ht][4][i], acc[ht][5][i], acc[ht][6][i], acc[ht][7][i]);
      }
    }
  }
}

// One block per (request, query head).  One wave turns the splits' (m, l)
// into weights w_s = 2^(m_s - M) / sum_s' 2^(m_s' - M) l_s' (0 for an empty
// split) in LDS; then every thread sums w_s acc_s for its channels with all
// loads unconditional, so they are issued back to back.
constexpr int kMaxSplits = 4096;  // splits * pages per split covers 65536 pages at 16 per split

// Few splits (the common case): every thread loads all (m, l) pairs of its
// (request, head) and four acc columns of every split at once, so the merge
// takes one memory round trip and no barrier.  Indices past nsplit are
// clamped and masked.  A 128-thread block takes 128 / (DV / 4) heads (four at
// DV = 128), so that no thread idles.
constexpr int kMergeFew = 16;
constexpr int kMergeThreads = 128;

template <int NS>
__global__ __launch_bounds__(kMergeThreads) void merge_few_kernel(const float* __restrict__ part_acc,
                                                                  const float* __restrict__ part_ml,
                                                                  float* __restrict__ out, int nsplit, int DV,
                                                                  int64_t nheads) {
  const int tph = DV / 4;  // threads per head
  const int hpb = tph < kMergeThreads ? kMergeThreads / tph : 1;
  const int64_t bh = (int64_t)blockIdx.x * hpb + threadIdx.x / tph;
  if (bh >= nheads) return;
  const float* ml = part_ml + bh * nsplit * 2;
  const float* acc = part_acc + bh * nsplit * DV;
  for (int c = 4 * (threadIdx.x % tph); c < DV; c += 4 * (tph < kMergeThreads ? tph : kMergeThreads)) {
    float m[NS], l[NS];
    float4 v[NS];
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      const int s = min(sp, nsplit - 1);
      m[sp] = ml[2 * s];
      l[sp] = ml[2 * s + 1];
      v[sp] = *reinterpret_cast<const float4*>(acc + (int64_t)s * DV + c);
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) M = fmaxf(M, m[sp]);
    float den = 0.f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      // an empty split (m = -inf) never wrote its acc; a clamped duplicate
      // (sp >= nsplit) is not counted
      const bool live = sp < nsplit && m[sp] != -__builtin_inff();
      const float wgt = live ? __builtin_amdgcn_exp2f(m[sp] - M) : 0.f;
      den += wgt * l[sp];
      num.x += live ? wgt * v[sp].x : 0.f;
      num.y += live ? wgt * v[sp].y : 0.f;
      num.z += live ? wgt * v[sp].z : 0.f;
      num.w += live ? wgt * v[sp].w : 0.f;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    float* o = out + bh * DV + c;
    if ((reinterpret_cast<uintptr_t>(out) & 15) == 0) {
      *reinterpret_cast<float4*>(o) = make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
    } else {  // the output need only be 4-byte aligned
      o[0] = num.x * inv;
      o[1] = num.y * inv;
      o[2] = num.z * inv;
      o[3] = num.w * inv;
    }
  }
}

// Many splits: one block per (request, query head), weights through LDS as
// described above.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_acc,
                                                    const float* __restrict__ part_ml, float* __restrict__ out,
                                                    int nsplit, int DV) {
  __shared__ float wts[kMaxSplits];
  const int64_t bh = blockIdx.x;
  const float* ml = part_ml + bh * nsplit * 2;
  const float* acc = part_acc + bh * nsplit * DV;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    float M = -__builtin_inff();
    for (int sp = lane; sp < nsplit; sp += kWave) M = fmaxf(M, ml[2 * sp]);
    M = wave_max(M);
    float den = 0.f;
    for (int sp = lane; sp < nsplit; sp += kWave) {
      const float m = ml[2 * sp];
      den += m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - M) * ml[2 * sp + 1];
    }
    den = wave_sum(den);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int sp = lane; sp < nsplit; sp += kWave) {
      const float m = ml[2 * sp];
      wts[sp] = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - M) * inv;
    }
  }
  __syncthreads();
  // an empty split never wrote its acc: its weight is 0 and its acc is not used
  auto term = [&](int sp, float a) { return wts[sp] != 0.f ? wts[sp] * a : 0.f; };
  for (int c = threadIdx.x; c < DV; c += blockDim.x) {
    float num = 0.f;
    int sp = 0;
    for (; sp + 4 <= nsplit; sp += 4) {
      const float a0 = acc[(int64_t)sp * DV + c], a1 = acc[(int64_t)(sp + 1) * DV + c];
      const float a2 = acc[(int64_t)(sp + 2) * DV + c], a3 = acc[(int64_t)(sp + 3) * DV + c];
      num += (term(sp, a0) + term(sp + 1, a1)) + (term(sp + 2, a2) + term(sp + 3, a3));
    }
    for (; sp < nsplit; ++sp) num += term(sp, acc[(int64_t)sp * DV + c]);
    out[bh * DV + c] = num;
  }
}

// The split merge for DV channels per head: few splits pack several heads
// into a block; many splits take the LDS path.
static hipError_t launch_merge(const DecodeArgs& a, int DV, hipStream_t st) {
  const int64_t nheads = (int64_t)a.B * a.Hq;
  if (a.splits > kMergeFew) {
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)nheads), dim3(128), 0, st, a.part_acc, a.part_ml, a.out, a.splits,
                       DV);
    return hipGetLastError();
  }
  const int tph = DV / 4;
  const int hpb = tph < kMergeThreads ? kMergeThreads / tph : 1;
  const dim3 grid((unsigned)((nheads + hpb - 1) / hpb));
#define SE_M(NS)                                                                                                   \
  if (a.splits <= NS) {                                                                                            \
    hipLaunchKernelGGL(merge_few_kernel<NS>, grid, dim3(kMergeThreads), 0, st, a.part_acc, a.part_ml, a.out,        \
                       a.splits, DV, nheads);                                                                      \
    return hipGetLastError();                                                                                      \
  }
  SE_M(2) SE_M(4) SE_M(8) SE_M(16)
#undef SE_M
  return hipErrorInvalidValue;
}

static bool mfma_decode_shape(const Layout& L, int G, bool valu) {
  return L.dk == 128 && L.dv == 128 && !L.visk && G <= 16 && !valu;
}

static bool mla_decode_shape(const Layout& L, int G, bool valu) {
  return L.dk == 576 && L.dv == 512 && L.visk && G <= 32 && !valu;
}

int decode_max_pps(const Layout& L, int G, bool valu) {
  if (mfma_decode_shape(L, G, valu)) return G <= 8 ? 256 : 128;
  if (mla_decode_shape(L, G, valu)) return kMlaPagesPerSplit;
  return (L.dk <= 128 && G <= 16) ? 32 : 16;
}

int decode_splits(const Layout& L, int B, int Hq, int MP, int topk, bool dense, int requested, bool valu) {
  // pages attended per (request, KV head) at most
  const int kmax = (dense || topk >= MP) ? MP : topk;
  if (kmax <= 0) return 1;
  const int units = B * L.hkv;
  const int G = Hq / L.hkv;
  const int mp = decode_max_pps(L, G, valu);
  const int smin = (kmax + mp - 1) / mp;
  // about one block per CU for the matrix-core GQA decode (measured at 128K,
  // 256 kept pages: 2 splits = 256 blocks 54.3 us with the merge, 4 splits =
  // 512 blocks 57.0 us, 1 split = 128 blocks 55.6 us without a merge: half the
  // CUs idle), one full round of resident blocks for the others (x 4 for the
  // VALU kernel); more splits only add per-block latency and merge traffic, a
  // partial second round idles the chip
  const int target = mla_decode_shape(L, G, valu) ? kMlaTargetBlocks / ((G + kMlaHeadsPerBlock - 1) / kMlaHeadsPerBlock)
                     : mfma_decode_shape(L, G, valu) ? 256 : 1024;
  int s = requested > 0 ? requested : (target + units - 1) / units;
  // the matrix-core GQA decode keeps at least 32 pages (8 per wave) per split
  // while that still gives every CU a block: fewer leave each block with more
  // fixed cost than streaming (measured at 32K, 128 kept pages: 23.0 us with 4
  // splits, 28.5 us with 8)
  if (requested <= 0 && mfma_decode_shape(L, G, valu)) {
    const int s32 = kmax / 32 > 0 ? kmax / 32 : 1;
    if ((int64_t)units * s32 >= 256 && s > s32) s = s32;
  }
  if (s < smin) s = smin;
  if (s > kmax) s = kmax;
  if (s > kMaxSplits) s = kMaxSplits;
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
  return launch_merge(a, DV, st);
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

template <int G>
static hipError_t launch_mfma_g(const Layout& L, const DecodeArgs& a, int pps, hipStream_t st) {
  const float scale2 = a.scale * kLog2e;
  dim3 grid(a.splits, L.hkv, a.B);
  if (a.splits == 1) {
    // one block per (KV head, request) writes the output itself: no merge
    hipLaunchKernelGGL((decode_mfma_kernel<G, 4, true>), grid, dim3(256), 0, st, a, L.hkv, L.ps, L.hs, L.ts, pps,
                       scale2);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_mfma_kernel<G, 4, false>), grid, dim3(256), 0, st, a, L.hkv, L.ps, L.hs, L.ts, pps,
                     scale2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(a, 128, st);
}

static hipError_t launch_mla(const Layout& L, const DecodeArgs& a, int pps, hipStream_t st) {
  const float scale2 = a.scale * kLog2e;
  const int nhb = (a.Hq / L.hkv + kMlaHeadsPerBlock - 1) / kMlaHeadsPerBlock;
  // two halves of the splits when their count is even: the first half,
  // dispatched first and so older on its CUs, takes longer splits
  const int kmax = a.selected ? (a.topk < a.MP ? a.topk : a.MP) : a.MP;
  int halves = 1, p0 = pps, p1 = pps;
  if (kMlaSplitTilt > 0 && a.splits % 2 == 0) {
    const int nsh = a.splits / 2;
    p1 = (int)((int64_t)kmax * 1024 / ((int64_t)nsh * (2048 + kMlaSplitTilt)));
    p0 = (kmax - nsh * p1 + nsh - 1) / nsh;
    if (p1 >= 1 && p0 <= kMlaPagesPerSplit) {
      halves = 2;
    } else {
      p0 = p1 = pps;
    }
  }
  dim3 grid(a.splits / halves * nhb, L.hkv, a.B * halves);
  // 16 heads per block, a four-page register ring (one pair in flight while
  // one is processed), two waves per SIMD (measured: 35.8 us against 38.7 us
  // for one 32-head block with a six-page ring at one wave per SIMD)
  hipLaunchKernelGGL((decode_mla_kernel<1, 4, 2>), grid, dim3(256), 0, st, a, L.hkv, L.ps, L.hs, L.ts, p0, p1, scale2,
                     nhb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(a, 512, st);
}

// Decode path: the matrix-core kernels for Dk = Dv = 128 with G <= 16 and for
// the MLA layout with G <= 32, unless the caller asks for the vector-ALU
// kernel (valu); the vector-ALU kernel for every other shape.
hipError_t launch_decode(const Layout& L, const DecodeArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / L.hkv;
  const int kmax = a.selected ? (a.topk < a.MP ? a.topk : a.MP) : a.MP;
  const int pps = (kmax + a.splits - 1) / a.splits;
  if (pps > decode_max_pps(L, G, a.valu)) return hipErrorInvalidValue;  // the host checks this before any launch
  if (mfma_decode_shape(L, G, a.valu)) {
    switch (G) {
      case 1: return launch_mfma_g<1>(L, a, pps, st);
      case 2: return launch_mfma_g<2>(L, a, pps, st);
      case 4: return launch_mfma_g<4>(L, a, pps, st);
      case 8: return launch_mfma_g<8>(L, a, pps, st);
      case 16: return launch_mfma_g<16>(L, a, pps, st);
      default: break;
    }
  }
  if (mla_decode_shape(L, G, a.valu)) return launch_mla(L, a, pps, st);
  if (L.dk == 64 && L.dv == 64 && !L.visk) return launch_d<64, 64, false>(L, a, G, pps, st);
  if (L.dk == 128 && L.dv == 128 && !L.visk) return launch_d<128, 128, false>(L, a, G, pps, st);
  if (L.dk == 576 && L.dv == 512 && L.visk) return launch_d<576, 512, true>(L, a, G, pps, st);
  return hipErrorInvalidValue;
}

}  // namespace se
