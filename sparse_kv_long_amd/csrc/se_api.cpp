// C ABI of the sparse-KV library: argument validation, workspace carving and
// the launch sequence of each entry point.  Every check runs on the host
// before anything is enqueued, so a call that fails writes nothing.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <new>

#include "../../include/se.h"
#include "se_internal.h"

namespace {

using se::Layout;

constexpr int kVersion = 400;  // 0.4.0: explicit vector-ALU attention switch in se_decode_params

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool pow2_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32; }

int check_layout(const se_kv_layout* L) {
  if (!L) return SE_EINVAL;
  if (L->reserved != 0) return SE_EINVAL;
  if (L->page_size != SE_PAGE_SIZE) return SE_EUNSUPPORTED;
  if (L->num_kv_heads < 1) return SE_EINVAL;
  if (L->v_is_k_prefix != 0 && L->v_is_k_prefix != 1) return SE_EINVAL;
  const bool ok_dims = (L->head_dim_qk == 64 && L->head_dim_v == 64 && !L->v_is_k_prefix) ||
                       (L->head_dim_qk == 128 && L->head_dim_v == 128 && !L->v_is_k_prefix) ||
                       (L->head_dim_qk == 576 && L->head_dim_v == 512 && L->v_is_k_prefix);
  if (!ok_dims) return SE_EUNSUPPORTED;
  if (L->page_stride <= 0 || L->head_stride <= 0 || L->token_stride <= 0) return SE_EINVAL;
  if (L->page_stride % 8 || L->head_stride % 8 || L->token_stride % 8) return SE_EINVAL;
  if (L->token_stride < L->head_dim_qk) return SE_EINVAL;
  return SE_OK;
}

Layout to_layout(const se_kv_layout* L) {
  Layout o;
  o.hkv = L->num_kv_heads;
  o.dk = L->head_dim_qk;
  o.dv = L->head_dim_v;
  o.visk = L->v_is_k_prefix;
  o.ps = L->page_stride;
  o.hs = L->head_stride;
  o.ts = L->token_stride;
  return o;
}

// pages a (request, KV head) keeps at most: the selected budget plus the forced pages
int kept_cap(const se_decode_params* p) { return p->topk + p->sink_pages + p->recent_pages; }

int check_counts(const se_decode_params* p) {
  if (p->topk < 0 || p->sink_pages < 0 || p->recent_pages < 0) return SE_EINVAL;
  if (p->topk > 65536 || p->sink_pages > 65536 || p->recent_pages > 65536) return SE_EUNSUPPORTED;
  if (kept_cap(p) < 1) return SE_EINVAL;
  if (p->topk == 0 && p->refresh_last_page) return SE_EINVAL;  // nothing is scored, so nothing to refresh for
  return SE_OK;
}

int check_params(const se_kv_layout* L, const se_decode_params* p) {
  if (!p) return SE_EINVAL;
  if (p->batch < 0 || p->num_q_heads < 1 || p->max_pages_per_seq < 1) return SE_EINVAL;
  if (const int rc = check_counts(p)) return rc;
  if (p->num_q_heads % L->num_kv_heads) return SE_EINVAL;
  if (!pow2_group(p->num_q_heads / L->num_kv_heads)) return SE_EUNSUPPORTED;
  if (p->max_pages_per_seq > 65536) return SE_EUNSUPPORTED;
  if (!(p->sm_scale >= 0.f) || isinf(p->sm_scale)) return SE_EINVAL;
  if (p->head_agg != 0 && p->head_agg != 1) return SE_EINVAL;
  if (p->refresh_last_page != 0 && p->refresh_last_page != 1) return SE_EINVAL;
  if (p->num_splits < 0) return SE_EINVAL;
  if (p->valu_attention != 0 && p->valu_attention != 1) return SE_EINVAL;
  return SE_OK;
}

float eff_scale(const se_kv_layout* L, const se_decode_params* p) {
  return p->sm_scale > 0.f ? p->sm_scale : 1.f / sqrtf((float)L->head_dim_qk);
}

struct DecodeWs {
  size_t scores, sel, phys, acc, ml, total;
  int splits;
  bool fits;  // every split holds no more pages than its kernel can stage
};

DecodeWs decode_ws(const se_kv_layout* L, const se_decode_params* p, bool dense) {
  const Layout l = to_layout(L);
  DecodeWs w;
  const int B = p->batch, Hkv = L->num_kv_heads, MP = p->max_pages_per_seq;
  const bool valu = p->valu_attention != 0;
  w.splits = se::decode_splits(l, B, p->num_q_heads, MP, kept_cap(p), dense, p->num_splits, valu);
  const int s_other = se::decode_splits(l, B, p->num_q_heads, MP, kept_cap(p), !dense, p->num_splits, valu);
  const int smax = w.splits > s_other ? w.splits : s_other;
  w.scores = 0;
  w.sel = w.scores + align256((size_t)B * Hkv * MP * sizeof(float));
  w.phys = w.sel + align256((size_t)B * Hkv * kept_cap(p) * sizeof(int32_t));
  w.acc = w.phys + align256((size_t)B * Hkv * kept_cap(p) * sizeof(int32_t));
  w.ml = w.acc + align256((size_t)B * p->num_q_heads * smax * L->head_dim_v * sizeof(float));
  w.total = w.ml + align256((size_t)B * p->num_q_heads * smax * 2 * sizeof(float));
  // pages per split of the chosen split count, for the dense and the sparse
  // page count, against what one block of the chosen kernel stages
  const int G = p->num_q_heads / Hkv, mp = se::decode_max_pps(l, G, valu);
  const int kd = MP, ks = kept_cap(p) < MP ? kept_cap(p) : MP;
  const int k_this = dense ? kd : ks, k_other = dense ? ks : kd;
  w.fits = (k_this + w.splits - 1) / w.splits <= mp && (k_other + s_other - 1) / s_other <= mp;
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SE_OK : SE_EHIP; }

// Row length of kept_idx: the most positions any prompt length up to
// max_prompt_len can keep, max(sink, ib) + budget + max(recent, window, N - ie).
int64_t snap_kept_capacity(const se_snapkv_params* p) {
  const bool iv = p->interval_end != 0;
  const int64_t ib = iv ? p->interval_begin : 0, ie = iv ? p->interval_end : p->max_prompt_len;
  int64_t tail = p->recent > p->window ? p->recent : p->window;
  if (p->max_prompt_len - ie > tail) tail = p->max_prompt_len - ie;
  return (p->sink > ib ? p->sink : ib) + (int64_t)p->budget + tail;
}

int check_snap(const se_snapkv_params* p) {
  if (!p) return SE_EINVAL;
  if (p->batch < 0 || p->num_kv_heads < 1 || p->num_q_heads < 1 || p->max_prompt_len < 1) return SE_EINVAL;
  if (p->num_q_heads % p->num_kv_heads) return SE_EINVAL;
  if (p->num_q_heads / p->num_kv_heads > 32) return SE_EUNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return SE_EUNSUPPORTED;
  if (p->window < 1 || p->budget < 1) return SE_EINVAL;
  if (p->window > 128) return SE_EUNSUPPORTED;
  if (p->pool_kernel < 1 || p->pool_kernel % 2 == 0) return SE_EINVAL;
  if (p->pool_kernel > se::kMaxPoolKernel) return SE_EUNSUPPORTED;
  if (p->sink < 0 || p->recent < 0) return SE_EINVAL;
  if (p->interval_end != 0 &&
      (p->interval_begin < 0 || p->interval_begin >= p->interval_end || p->interval_end > p->max_prompt_len))
    return SE_EINVAL;
  if (p->interval_end == 0 && p->interval_begin != 0) return SE_EINVAL;
  if (p->max_prompt_len - p->window > 65536) return SE_EUNSUPPORTED;
  if (snap_kept_capacity(p) > INT32_MAX / 2) return SE_EINVAL;
  if (p->out_capacity < snap_kept_capacity(p)) return SE_EINVAL;
  if (!(p->sm_scale >= 0.f) || isinf(p->sm_scale)) return SE_EINVAL;
  return SE_OK;
}

se::SnapArgs snap_args(const se_snapkv_params* p, const void* q_win, const void* k, const void* v,
                       const int32_t* lens) {
  se::SnapArgs a;
  a.q_win = static_cast<const uint16_t*>(q_win);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.lens = lens;
  a.B = p->batch;
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.D = p->head_dim;
  a.N = p->max_prompt_len;
  a.W = p->window;
  a.pool = p->pool_kernel;
  a.R = p->budget;
  a.cap = p->out_capacity;
  a.sink = p->sink;
  a.rec = p->recent > p->window ? p->recent : p->window;
  a.ib = p->interval_end != 0 ? p->interval_begin : 0;
  a.ie = p->interval_end != 0 ? p->interval_end : p->max_prompt_len;
  a.kcap = (int)snap_kept_capacity(p);
  a.scale = p->sm_scale > 0.f ? p->sm_scale : 1.f / sqrtf((float)p->head_dim);
  return a;
}

int check_decode_ptrs(const se_kv_layout* layout, const void* q, const void* k_pages, const void* v_pages,
                             const int32_t* page_table, const int32_t* seq_lens, const float* out) {
  if (!q || !k_pages || !page_table || !seq_lens || !out) return SE_EINVAL;
  if (!layout->v_is_k_prefix && !v_pages) return SE_EINVAL;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(out)) return SE_EINVAL;
  if (!layout->v_is_k_prefix && !aligned16(v_pages)) return SE_EINVAL;
  return SE_OK;
}

}  // namespace

namespace se {

int sparse_decode_check(const se_kv_layout* layout, const se_decode_params* params, const void* q,
                        const void* k_pages, const void* v_pages, const int32_t* page_table, const void* summaries,
                        const int32_t* seq_lens, const float* out, size_t* need) {
  *need = 0;
  int rc = check_layout(layout);
  if (rc) return rc;
  rc = check_params(layout, params);
  if (rc) return rc;
  if (params->batch == 0) return SE_OK;
  rc = check_decode_ptrs(layout, q, k_pages, v_pages, page_table, seq_lens, out);
  if (rc) return rc;
  const bool all_dense = kept_cap(params) >= params->max_pages_per_seq;
  // topk = 0 (sink and recent pages only) scores nothing
  const bool need_scores = (!all_dense && params->topk > 0) || params->refresh_last_page;
  if (need_scores && (!summaries || !aligned16(summaries))) return SE_EINVAL;
  const DecodeWs w = decode_ws(layout, params, all_dense);
  if (!w.fits) return SE_EUNSUPPORTED;
  *need = w.total;
  return SE_OK;
}

int sparse_decode_enqueue(const se_kv_layout* layout, const se_decode_params* params, const void* q,
                          const void* k_pages, const void* v_pages, const int32_t* page_table, void* summaries,
                          const int32_t* seq_lens, float* out, int32_t* selected, void* workspace, hipStream_t st) {
  int rc = SE_OK;
  const int kcap = kept_cap(params);
  const bool all_dense = kcap >= params->max_pages_per_seq;
  const bool need_scores = (!all_dense && params->topk > 0) || params->refresh_last_page;
  const DecodeWs w = decode_ws(layout, params, all_dense);
  const Layout L = to_layout(layout);
  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws + w.scores);
  int32_t* sel = selected ? selected : reinterpret_cast<int32_t*>(ws + w.sel);
  int32_t* phys = reinterpret_cast<int32_t*>(ws + w.phys);
  const float scale = eff_scale(layout, params);

  if (need_scores) {
    se::ScoreArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k_pages);
    a.page_table = page_table;
    a.summ = static_cast<uint16_t*>(summaries);
    a.seq_lens = seq_lens;
    a.scores = scores;
    a.B = params->batch;
    a.Hq = params->num_q_heads;
    a.MP = params->max_pages_per_seq;
    a.topk = kcap;  // a request with kcap >= its pages runs dense and is not scored
    a.refresh = params->refresh_last_page;
    a.head_sum = params->head_agg;
    a.scale = scale;
    rc = hip_status(se::launch_quest_scores(L, a, st));
    if (rc) return rc;
  }
  if (!all_dense || selected) {
    rc = hip_status(se::launch_topk_pages(params->batch, L.hkv, params->max_pages_per_seq, params->topk,
                                          params->sink_pages, params->recent_pages, scores, seq_lens, sel, page_table,
                                          all_dense ? nullptr : phys, st));
    if (rc) return rc;
  }
  se::DecodeArgs d;
  d.q = static_cast<const uint16_t*>(q);
  d.k = static_cast<const uint16_t*>(k_pages);
  d.v = static_cast<const uint16_t*>(v_pages);
  d.page_table = page_table;
  d.seq_lens = seq_lens;
  d.selected = all_dense ? nullptr : sel;
  d.selected_phys = all_dense ? nullptr : phys;
  d.out = out;
  d.part_acc = reinterpret_cast<float*>(ws + w.acc);
  d.part_ml = reinterpret_cast<float*>(ws + w.ml);
  d.B = params->batch;
  d.Hq = params->num_q_heads;
  d.MP = params->max_pages_per_seq;
  d.topk = kcap;  // row length of the selection
  d.splits = w.splits;
  d.scale = scale;
  d.valu = params->valu_attention != 0;
  return hip_status(se::launch_decode(L, d, st));
}

}  // namespace se

extern "C" {

int se_version(void) { return kVersion; }

const char* se_status_string(int status) {
  switch (status) {
    case SE_OK: return "ok";
    case SE_EINVAL: return "invalid argument";
    case SE_EUNSUPPORTED: return "unsupported configuration";
    case SE_EWORKSPACE: return "workspace missing or too small";
    case SE_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int se_build_summaries(const se_kv_layout* layout, int32_t batch, int32_t max_pages_per_seq, const void* k_pages,
                       const int32_t* page_table, const int32_t* seq_lens, void* summaries, void* stream) {
  int rc = check_layout(layout);
  if (rc) return rc;
  if (batch < 0 || max_pages_per_seq < 1) return SE_EINVAL;
  if (batch == 0) return SE_OK;
  if (!k_pages || !page_table || !seq_lens || !summaries) return SE_EINVAL;
  if (!aligned16(k_pages) || !aligned16(summaries)) return SE_EINVAL;
  return hip_status(se::launch_build_summaries(to_layout(layout), batch, max_pages_per_seq,
                                               static_cast<const uint16_t*>(k_pages), page_table, seq_lens,
                                               static_cast<uint16_t*>(summaries), (hipStream_t)stream));
}

int se_sparse_decode_workspace_size(const se_kv_layout* layout, const se_decode_params* params, size_t* bytes) {
  int rc = check_layout(layout);
  if (rc) return rc;
  rc = check_params(layout, params);
  if (rc) return rc;
  if (!bytes) return SE_EINVAL;
  const DecodeWs w = decode_ws(layout, params, kept_cap(params) >= params->max_pages_per_seq);
  if (!w.fits) return SE_EUNSUPPORTED;
  *bytes = w.total;
  return SE_OK;
}


int se_sparse_decode(const se_kv_layout* layout, const se_decode_params* params, const void* q, const void* k_pages,
                     const void* v_pages, const int32_t* page_table, void* summaries, const int32_t* seq_lens,
                     float* out, int32_t* selected, void* workspace, size_t workspace_bytes, void* stream) {
  size_t need = 0;
  const int rc = se::sparse_decode_check(layout, params, q, k_pages, v_pages, page_table, summaries, seq_lens, out,
                                         &need);
  if (rc) return rc;
  if (params->batch == 0) return SE_OK;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return SE_EWORKSPACE;
  return se::sparse_decode_enqueue(layout, params, q, k_pages, v_pages, page_table, summaries, seq_lens, out, selected,
                                   workspace, (hipStream_t)stream);
}

int se_quest_scores(const se_kv_layout* layout, const se_decode_params* params, const void* q, const void* k_pages,
                    const int32_t* page_table, void* summaries, const int32_t* seq_lens, float* scores,
                    void* stream) {
  int rc = check_layout(layout);
  if (rc) return rc;
  rc = check_params(layout, params);
  if (rc) return rc;
  if (params->batch == 0) return SE_OK;
  if (!q || !k_pages || !page_table || !summaries || !seq_lens || !scores) return SE_EINVAL;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(summaries)) return SE_EINVAL;
  se::ScoreArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_pages);
  a.page_table = page_table;
  a.summ = static_cast<uint16_t*>(summaries);
  a.seq_lens = seq_lens;
  a.scores = scores;
  a.B = params->batch;
  a.Hq = params->num_q_heads;
  a.MP = params->max_pages_per_seq;
  a.topk = kept_cap(params);  // a request with kcap >= its pages runs dense and is not scored
  a.refresh = params->refresh_last_page;
  a.head_sum = params->head_agg;
  a.scale = eff_scale(layout, params);
  return hip_status(se::launch_quest_scores(to_layout(layout), a, (hipStream_t)stream));
}

int se_topk_pages(const se_decode_params* params, int32_t num_kv_heads, const float* scores, const int32_t* seq_lens,
                  int32_t* selected, void* stream) {
  if (!params || num_kv_heads < 1) return SE_EINVAL;
  if (params->batch < 0 || params->max_pages_per_seq < 1) return SE_EINVAL;
  if (const int rc = check_counts(params)) return rc;
  if (params->max_pages_per_seq > 65536) return SE_EUNSUPPORTED;
  if (params->batch == 0) return SE_OK;
  if ((params->topk > 0 && !scores) || !seq_lens || !selected) return SE_EINVAL;
  return hip_status(se::launch_topk_pages(params->batch, num_kv_heads, params->max_pages_per_seq, params->topk,
                                          params->sink_pages, params->recent_pages, scores, seq_lens, selected,
                                          nullptr, nullptr, (hipStream_t)stream));
}

int se_decode_selected(const se_kv_layout* layout, const se_decode_params* params, const void* q, const void* k_pages,
                       const void* v_pages, const int32_t* page_table, const int32_t* seq_lens,
                       const int32_t* selected, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_layout(layout);
  if (rc) return rc;
  rc = check_params(layout, params);
  if (rc) return rc;
  if (params->batch == 0) return SE_OK;
  rc = check_decode_ptrs(layout, q, k_pages, v_pages, page_table, seq_lens, out);
  if (rc) return rc;
  const bool dense = selected == nullptr;
  const DecodeWs w = decode_ws(layout, params, dense);
  if (!w.fits) return SE_EUNSUPPORTED;
  if (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 255u)) return SE_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  se::DecodeArgs d;
  d.q = static_cast<const uint16_t*>(q);
  d.k = static_cast<const uint16_t*>(k_pages);
  d.v = static_cast<const uint16_t*>(v_pages);
  d.page_table = page_table;
  d.seq_lens = seq_lens;
  d.selected = selected;
  d.selected_phys = nullptr;
  d.out = out;
  d.part_acc = reinterpret_cast<float*>(ws + w.acc);
  d.part_ml = reinterpret_cast<float*>(ws + w.ml);
  d.B = params->batch;
  d.Hq = params->num_q_heads;
  d.MP = params->max_pages_per_seq;
  d.topk = kept_cap(params);  // row length of the selection
  d.splits = w.splits;
  d.scale = eff_scale(layout, params);
  d.valu = params->valu_attention != 0;
  return hip_status(se::launch_decode(to_layout(layout), d, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
int se_snapkv_workspace_size(const se_snapkv_params* params, size_t* bytes) {
  const int rc = check_snap(params);
  if (rc) return rc;
  if (!bytes) return SE_EINVAL;
  *bytes = se::snap_workspace_bytes(snap_args(params, nullptr, nullptr, nullptr, nullptr));
  return SE_OK;
}

static int check_ws(const se::SnapArgs& a, void* ws, size_t bytes) {
  if (!ws || bytes < se::snap_workspace_bytes(a) || ((uintptr_t)ws & 255u)) return SE_EWORKSPACE;
  return SE_OK;
}

int se_snapkv_kept_capacity(const se_snapkv_params* params, int32_t* kcap) {
  const int rc = check_snap(params);
  if (rc) return rc;
  if (!kcap) return SE_EINVAL;
  *kcap = (int32_t)snap_kept_capacity(params);
  return SE_OK;
}

// [a, a + na) and [b, b + nb) share a byte
static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// The compaction reads rows of k/v while it writes k_out/v_out, so the two
// pairs must not share memory.
static bool outputs_overlap_inputs(const se_snapkv_params* p, const void* k, const void* v, const void* k_out,
                                   const void* v_out) {
  const size_t in_bytes = (size_t)p->batch * p->num_kv_heads * p->max_prompt_len * p->head_dim * 2;
  const size_t out_bytes = (size_t)p->batch * p->num_kv_heads * p->out_capacity * p->head_dim * 2;
  return overlaps(k, in_bytes, k_out, out_bytes) || overlaps(k, in_bytes, v_out, out_bytes) ||
         overlaps(v, in_bytes, k_out, out_bytes) || overlaps(v, in_bytes, v_out, out_bytes);
}

static int snap_evict(const se_snapkv_params* params, const void* q_win, const void* k, const void* v,
                      const int32_t* prompt_lens, const int32_t* positions, void* k_out, void* v_out,
                      int32_t* kept_idx, int32_t* kept_len, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_snap(params);
  if (rc) return rc;
  if (params->batch == 0) return SE_OK;
  if (!q_win || !k || !v || !prompt_lens || !k_out || !v_out || !kept_idx || !kept_len) return SE_EINVAL;
  if (!aligned16(q_win) || !aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out)) return SE_EINVAL;
  if (outputs_overlap_inputs(params, k, v, k_out, v_out)) return SE_EINVAL;
  const se::SnapArgs a = snap_args(params, q_win, k, v, prompt_lens);
  rc = check_ws(a, workspace, workspace_bytes);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  const se::SnapWork w = se::snap_workspace_carve(a, workspace);
  rc = hip_status(se::launch_snap_votes(a, w, true, w.votes, st));
  if (rc) return rc;
  rc = hip_status(se::launch_maxpool(a, w.votes, se::snap_row_groups(a), w.pooled, true, st));
  if (rc) return rc;
  rc = hip_status(se::launch_snap_select(a, w.pooled, kept_idx, kept_len, st));
  if (rc) return rc;
  rc = hip_status(se::launch_compact(a, kept_idx, kept_len, static_cast<uint16_t*>(k_out),
                                     static_cast<uint16_t*>(v_out), st));
  if (rc || !positions) return rc;
  return hip_status(se::launch_map_positions(a, positions, kept_idx, kept_len, st));
}

int se_snapkv_compact(const se_snapkv_params* params, const void* q_win, const void* k, const void* v,
                      const int32_t* prompt_lens, void* k_out, void* v_out, int32_t* kept_idx, int32_t* kept_len,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return snap_evict(params, q_win, k, v, prompt_lens, nullptr, k_out, v_out, kept_idx, kept_len, workspace,
                    workspace_bytes, stream);
}

int se_snapkv_recompact(const se_snapkv_params* params, const void* q_win, const void* k, const void* v,
                        const int32_t* cache_lens, const int32_t* positions, void* k_out, void* v_out,
                        int32_t* kept_idx, int32_t* kept_len, void* workspace, size_t workspace_bytes, void* stream) {
  if (params && params->batch > 0 && !positions) return SE_EINVAL;
  return snap_evict(params, q_win, k, v, cache_lens, positions, k_out, v_out, kept_idx, kept_len, workspace,
                    workspace_bytes, stream);
}

int se_pyramid_budgets(int32_t num_layers, int32_t budget, double ratio_first, double ratio_last,
                       int32_t* budgets) {
  if (!budgets || num_layers < 1 || budget < 1) return SE_EINVAL;
  if (num_layers > 4096 || budget > (1 << 24)) return SE_EUNSUPPORTED;
  if (!(ratio_first > 0.0 && ratio_first <= 1000.0) || !(ratio_last > 0.0 && ratio_last <= 1000.0))
    return SE_EINVAL;
  // ratios to nine decimals (round half to even), then exact integer shares
  const int64_t A = (int64_t)nearbyint(ratio_first * 1e9), Z = (int64_t)nearbyint(ratio_last * 1e9);
  if (A < 1 || Z < 1) return SE_EINVAL;
  const int L = num_layers;
  __int128 total_w = 0;
  for (int l = 0; l < L; ++l) total_w += L == 1 ? A : (__int128)A * (L - 1) + (__int128)(Z - A) * l;
  const __int128 tokens = (__int128)L * budget;
  __int128 given = 0;
  // floors of the exact shares; remainders kept for the leftover tokens
  __int128* rem = new (std::nothrow) __int128[L];
  if (!rem) return SE_EINVAL;
  for (int l = 0; l < L; ++l) {
    const __int128 w = L == 1 ? A : (__int128)A * (L - 1) + (__int128)(Z - A) * l;
    const __int128 share = tokens * w;
    budgets[l] = (int32_t)(share / total_w);
    rem[l] = share % total_w;
    given += budgets[l];
  }
  // one more token to each of the layers with the largest remainders, ties to the lower layer
  for (__int128 extra = tokens - given; extra > 0; --extra) {
    int best = -1;
    for (int l = 0; l < L; ++l)
      if (rem[l] >= 0 && (best < 0 || rem[l] > rem[best])) best = l;
    budgets[best] += 1;
    rem[best] = -1;
  }
  delete[] rem;
  return SE_OK;
}

int se_snapkv_votes(const se_snapkv_params* params, const void* q_win, const void* k, const int32_t* prompt_lens,
                    float* votes, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_snap(params);
  if (rc) return rc;
  if (params->batch == 0) return SE_OK;
  if (!q_win || !k || !prompt_lens || !votes) return SE_EINVAL;
  if (!aligned16(q_win) || !aligned16(k)) return SE_EINVAL;
  const se::SnapArgs a = snap_args(params, q_win, k, nullptr, prompt_lens);
  rc = check_ws(a, workspace, workspace_bytes);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  const se::SnapWork w = se::snap_workspace_carve(a, workspace);
  rc = hip_status(se::launch_snap_votes(a, w, false, w.votes, st));
  if (rc) return rc;
  // sum the row groups into the caller's array (a pool of width 1)
  se::SnapArgs a1 = a;
  a1.pool = 1;
  return hip_status(se::launch_maxpool(a1, w.votes, se::snap_row_groups(a), votes, false, st));
}

int se_maxpool1d(const se_snapkv_params* params, const float* votes, const int32_t* prompt_lens, float* pooled,
                 void* stream) {
  int rc = check_snap(params);
  if (rc) return rc;
  if (params->batch == 0) return SE_OK;
  if (!votes || !prompt_lens || !pooled) return SE_EINVAL;
  const se::SnapArgs a = snap_args(params, nullptr, nullptr, nullptr, prompt_lens);
  return hip_status(se::launch_maxpool(a, votes, 1, pooled, false, (hipStream_t)stream));
}

int se_snapkv_select(const se_snapkv_params* params, const float* pooled, const int32_t* prompt_lens,
                     int32_t* kept_idx, int32_t* kept_len, void* stream) {
  int rc = check_snap(params);
  if (rc) return rc;
  if (params->batch == 0) return SE_OK;
  if (!pooled || !prompt_lens || !kept_idx || !kept_len) return SE_EINVAL;
  const se::SnapArgs a = snap_args(params, nullptr, nullptr, nullptr, prompt_lens);
  return hip_status(se::launch_snap_select(a, pooled, kept_idx, kept_len, (hipStream_t)stream));
}

int se_compact(const se_snapkv_params* params, const void* k, const void* v, const int32_t* kept_idx,
               const int32_t* kept_len, void* k_out, void* v_out, void* stream) {
  int rc = check_snap(params);
  if (rc) return rc;
  if (params->batch == 0) return SE_OK;
  if (!k || !v || !kept_idx || !kept_len || !k_out || !v_out) return SE_EINVAL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out)) return SE_EINVAL;
  if (outputs_overlap_inputs(params, k, v, k_out, v_out)) return SE_EINVAL;
  const se::SnapArgs a = snap_args(params, nullptr, k, v, nullptr);
  return hip_status(se::launch_compact(a, kept_idx, kept_len, static_cast<uint16_t*>(k_out),
                                       static_cast<uint16_t*>(v_out), (hipStream_t)stream));
}

}  // extern "C"
