// Internal launch interface between the C ABI (se_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/se.h"

namespace se {

// se_sparse_decode in two halves.  sparse_decode_check runs every host-side
// check of the arguments except the workspace and sets *need to the
// workspace bytes the call takes (0 for an empty batch); sparse_decode_enqueue
// launches the step with a workspace of at least that many bytes, 256-byte
// aligned, on stream st (only after a successful check).
int sparse_decode_check(const se_kv_layout* layout, const se_decode_params* params, const void* q,
                        const void* k_pages, const void* v_pages, const int32_t* page_table, const void* summaries,
                        const int32_t* seq_lens, const float* out, size_t* need);
int sparse_decode_enqueue(const se_kv_layout* layout, const se_decode_params* params, const void* q,
                          const void* k_pages, const void* v_pages, const int32_t* page_table, void* summaries,
                          const int32_t* seq_lens, float* out, int32_t* selected, void* workspace, hipStream_t st);

struct Layout {
  int hkv, dk, dv, visk;
  int64_t ps, hs, ts;  // page, head and token strides in elements
};

// ---- Quest -----------------------------------------------------------------
hipError_t launch_build_summaries(const Layout& L, int B, int MP, const uint16_t* k, const int32_t* page_table,
                                  const int32_t* seq_lens, uint16_t* summ, hipStream_t st);

struct ScoreArgs {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* page_table;
  uint16_t* summ;
  const int32_t* seq_lens;
  float* scores;
  int B, Hq, MP, topk, refresh, head_sum;
  float scale;
};
hipError_t launch_quest_scores(const Layout& L, const ScoreArgs& a, hipStream_t st);

// Per (request, KV head): the first `sink` and last `recent` pages plus the
// `topk` best-scoring others; selected rows hold topk + sink + recent ids.
// phys (nullable): also write page_table[b][id] for every selected id.
// scores is not read when topk = 0.
hipError_t launch_topk_pages(int B, int Hkv, int MP, int topk, int sink, int recent, const float* scores,
                             const int32_t* seq_lens, int32_t* selected, const int32_t* page_table, int32_t* phys,
                             hipStream_t st);

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* selected;       // nullptr = dense
  const int32_t* selected_phys;  // physical ids of `selected`, or nullptr (looked up)
  float* out;
  float* part_acc;  // [B, Hq, S, Dv]
  float* part_ml;   // [B, Hq, S, 2]
  int B, Hq, MP, topk, splits;
  float scale;
  bool valu;  // vector-ALU attention kernel for every shape
};
// Split count of the attention over at most min(topk, MP) pages per (request,
// KV head) (every page when dense); `requested` > 0 asks for that many.
int decode_splits(const Layout& L, int B, int Hq, int MP, int topk, bool dense, int requested, bool valu);
// Most pages one split of the chosen attention kernel can hold.
int decode_max_pps(const Layout& L, int G, bool valu);
size_t decode_partials_bytes(const Layout& L, int B, int Hq, int splits);
hipError_t launch_decode(const Layout& L, const DecodeArgs& a, hipStream_t st);

// ---- SnapKV ----------------------------------------------------------------
constexpr int kMaxPoolKernel = 129;  // widest max-pool window the pooling kernel stages

struct SnapArgs {
  const uint16_t* q_win;  // [B, Hq, W, D]
  const uint16_t* k;      // [B, Hkv, N, D]
  const uint16_t* v;
  const int32_t* lens;
  int B, Hq, Hkv, D, N, W, pool, R, cap;
  int sink;  // leading positions always kept
  int rec;   // trailing positions always kept: max(recent, W)
  int ib;    // history interval [ib, ie) outside which nothing is dropped (0, N without one)
  int ie;
  int kcap;  // row length of kept_idx: max(sink, ib) + R + max(rec, N - ie)
  float scale;
};

// Positions a request of length n may drop: [lo, hi); hi - lo <= R means
// nothing is dropped (every position is kept).
__host__ __device__ inline void snap_candidates(const SnapArgs& a, int n, int& lo, int& hi) {
  lo = a.sink > a.ib ? a.sink : a.ib;
  hi = n - a.rec < a.ie ? n - a.rec : a.ie;
}
struct SnapWork {
  float* row_part;  // [B, Hkv, row_groups, nblk*waves, 128, 2] partial (max, sum)
  float* votes;     // [row_groups, B, Hkv, N]
  float* pooled;    // [B, Hkv, N]
};
size_t snap_workspace_bytes(const SnapArgs& a);
SnapWork snap_workspace_carve(const SnapArgs& a, void* ws);
// skip_kept: requests whose prefix already fits the budget are not scored.
hipError_t launch_snap_votes(const SnapArgs& a, const SnapWork& w, bool skip_kept, float* votes_out,
                             hipStream_t st);
hipError_t launch_maxpool(const SnapArgs& a, const float* votes, int row_groups, float* pooled,
                          bool skip_kept, hipStream_t st);
int snap_row_groups(const SnapArgs& a);
hipError_t launch_snap_select(const SnapArgs& a, const float* pooled, int32_t* kept_idx, int32_t* kept_len,
                              hipStream_t st);
hipError_t launch_compact(const SnapArgs& a, const int32_t* kept_idx, const int32_t* kept_len, uint16_t* k_out,
                          uint16_t* v_out, hipStream_t st);
// kept_idx[b][g][r] = positions[b][g][kept_idx[b][g][r]] for r < kept_len[b][g]
hipError_t launch_map_positions(const SnapArgs& a, const int32_t* positions, int32_t* kept_idx,
                                const int32_t* kept_len, hipStream_t st);

}  // namespace se
