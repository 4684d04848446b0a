/*
 * se.h -- C ABI of the MI355X (gfx950) sparse-KV decode library.
 *
 * Two method hooks, after the SparseEngine pages (arXiv 2609.39068):
 *
 *   Quest (query-aware page selection; Table 8: "16-token pages"): every
 *   16-token page of the paged KV cache carries a channel-wise min/max
 *   summary of its keys (Fig. 3: summaries attached to the KV blocks).  At
 *   each decode step every query head bounds each page's logits from the
 *   summary, the KV head keeps its top-k pages, and attention runs over the
 *   keys and values of those pages only.
 *
 *   SnapKV (prefill-side eviction; Table 8: "32 scoring window; pooling
 *   kernel 7"): the last W queries score the context, the scores are summed
 *   and max-pooled, the top R prefix tokens plus the window are kept, and
 *   the kept K/V rows are copied into a dense retained cache, so storage is
 *   really released (Table 15 note).  The same calls cover the eviction
 *   methods the pages configure around those scores: sink and recent tokens
 *   kept beside the selected budget (Tables 8-11), H2O (a 128-token scoring
 *   window, no pooling, a recent share of the budget), PyramidKV (per-layer
 *   budgets, se_pyramid_budgets), prefix-cache pruning inside a history
 *   interval (Figure 4) and re-eviction during decode (Tables 9-10:
 *   "eviction every 1,024 decode steps", se_snapkv_recompact).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer unless stated otherwise; the
 *    caller owns every buffer (KV pages, page table, summaries, outputs and
 *    workspace).  The library never allocates and keeps no state.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and returns without synchronising.  Device faults surface at the
 *    caller's next synchronisation.
 *  - bf16 is IEEE bfloat16 (the top 16 bits of an fp32).  Tensors are
 *    row-major; dims are listed outermost first.
 *  - Return value: SE_OK, or an error code.  Argument errors are detected on
 *    the host before anything is enqueued, so a failing call writes nothing.
 *    Contents of device arrays (lengths, page ids) are preconditions and are
 *    not checked.
 *  - Calls are thread-safe; calls that share output or workspace buffers
 *    must be ordered by the caller.
 */
#ifndef SPARSE_KV_SE_H_
#define SPARSE_KV_SE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SE_OK = 0,
  SE_EINVAL = 1,        /* null pointer, inconsistent sizes, bad value        */
  SE_EUNSUPPORTED = 2,  /* valid but not built: page size, head dims, group   */
  SE_EWORKSPACE = 3,    /* workspace missing or smaller than the size query   */
  SE_EHIP = 4           /* the HIP runtime refused a launch                   */
};

#define SE_PAGE_SIZE 16

/* Where the keys and values of a (page, KV head, token) live.
 *
 * Element address of channel c of token t of KV head g in page `pid`:
 *     base + pid*page_stride + g*head_stride + t*token_stride + c
 * The paged pool [P, Hkv, 16, D] has page_stride = Hkv*16*D,
 * head_stride = 16*D, token_stride = D.  A dense per-request cache
 * [B, Hkv, L, D] (L a multiple of 16) is read with page_stride = 16*D,
 * head_stride = L*D, token_stride = D and page id b*Hkv*L/16 + lp for
 * logical page lp of request b.
 * Strides are in elements, must be multiples of 8, and K and V share them.
 * Supported (head_dim_qk, head_dim_v): (64, 64), (128, 128), and (576, 512)
 * with v_is_k_prefix = 1 (latent attention: V is the first 512 channels of
 * the 576-channel key row, and v_pages is ignored).
 */
typedef struct se_kv_layout {
  int32_t page_size;      /* tokens per page; must be SE_PAGE_SIZE           */
  int32_t num_kv_heads;   /* Hkv                                              */
  int32_t head_dim_qk;    /* Dk                                               */
  int32_t head_dim_v;     /* Dv                                               */
  int32_t v_is_k_prefix;  /* 1: V = K[..., :Dv]                               */
  int32_t reserved;       /* must be 0                                        */
  int64_t page_stride;
  int64_t head_stride;
  int64_t token_stride;
} se_kv_layout;

typedef struct se_decode_params {
  int32_t batch;              /* B                                            */
  int32_t num_q_heads;        /* Hq, a multiple of Hkv; G = Hq/Hkv <= 32      */
  int32_t max_pages_per_seq;  /* row length of page_table (<= 65536)          */
  int32_t topk;               /* pages selected by score per (request, KV
                                 head), >= 0, beside the forced pages below.
                                 Request b runs dense when
                                 topk + sink_pages + recent_pages >= its pages. */
  float sm_scale;             /* softmax scale s; 0 means 1/sqrt(Dk)          */
  int32_t head_agg;           /* 0: page score = max over the KV head's query
                                 heads (default); 1: sum                      */
  int32_t refresh_last_page;  /* 1: recompute the summary of each request's
                                 last page from its keys before scoring      */
  int32_t num_splits;         /* split-K factor of the attention; 0 = auto    */
  int32_t sink_pages;         /* >= 0: the first sink_pages pages of every
                                 request are always kept                      */
  int32_t recent_pages;       /* >= 0: the last recent_pages pages of every
                                 request are always kept                      */
  int32_t valu_attention;     /* 0: the attention runs on the matrix cores
                                 where a kernel for the shape is built (Dk =
                                 Dv = 128 with G <= 16, and the 576/512 latent
                                 layout); 1: the vector-ALU dot-product kernel
                                 for every shape, which leaves the matrix
                                 cores to other work (slower here)           */
} se_decode_params;
/* Forced pages (SparseEngine appendix Tables 8-11: a sink and a recent budget
 * beside each method's selected budget, which excludes them; the StreamingLLM
 * rows keep sink and recent only).  A request keeps its forced pages plus the
 * topk best-scoring others, at most kcap = topk + sink_pages + recent_pages
 * pages; `selected` arrays are [B, Hkv, kcap].  topk = 0 is StreamingLLM: no
 * page is scored, `summaries` is not read (may be NULL) and refresh_last_page
 * must be 0.  kcap must be >= 1; each count <= 65536. */

/* Version as major*10000 + minor*100 + patch. */
int se_version(void);

/* Static description of a status code (never NULL). */
const char* se_status_string(int status);

/* ---------------------------------------------------------------------------
 * Quest, prefill side: page summaries.
 *
 * For every request b, valid logical page lp < ceil(seq_lens[b]/16) and KV
 * head g, writes summaries[page_table[b][lp]][g][0][:] = channel-wise min and
 * [1][:] = channel-wise max of the keys of the page's valid tokens
 * (t < seq_lens[b]).  min and max of bf16 values are bf16 values, so the
 * result is exact.  Pages past a request's length are not touched.
 *
 *   k_pages     bf16, addressed by `layout`
 *   page_table  int32 [batch, max_pages_per_seq]
 *   seq_lens    int32 [batch], each <= max_pages_per_seq*16
 *   summaries   bf16 [P, Hkv, 2, Dk], indexed by physical page id
 * ------------------------------------------------------------------------- */
int se_build_summaries(const se_kv_layout* layout, int32_t batch, int32_t max_pages_per_seq,
                       const void* k_pages, const int32_t* page_table, const int32_t* seq_lens,
                       void* summaries, void* stream);

/* ---------------------------------------------------------------------------
 * Quest, decode side: one attention layer's decode step for the batch.
 *
 *   q           bf16 [B, Hq, Dk]  (query of the current token)
 *   k_pages     bf16, `layout`;   v_pages bf16, `layout` (NULL if v_is_k_prefix)
 *   page_table  int32 [B, max_pages_per_seq]
 *   summaries   bf16 [P, Hkv, 2, Dk]; read, and with refresh_last_page the
 *               last page of each request is rewritten.  May be NULL only
 *               when refresh_last_page = 0 and either topk = 0 or
 *               kcap >= max_pages_per_seq.
 *   seq_lens    int32 [B]; counts the current token, whose K/V the caller
 *               has already appended.  0 gives a zero output row.
 *   out         fp32 [B, Hq, Dv]
 *   selected    int32 [B, Hkv, kcap] or NULL; receives each KV head's kept
 *               logical page ids in ascending order, padded with -1.
 *   workspace   device scratch of at least se_sparse_decode_workspace_size
 *               bytes, 256-byte aligned; contents need no initialisation.
 *
 * Steps: page scores (U = s * sum_c max(q_c*min_c, q_c*max_c) per query
 * head, reduced to the KV head), top-k per KV head (ties to the lower page
 * id) beside the forced sink and recent pages, split-K softmax attention over
 * the kept pages' valid tokens, and a log-sum-exp merge of the splits.
 * ------------------------------------------------------------------------- */
int se_sparse_decode_workspace_size(const se_kv_layout* layout, const se_decode_params* params,
                                    size_t* bytes);

int se_sparse_decode(const se_kv_layout* layout, const se_decode_params* params, const void* q,
                     const void* k_pages, const void* v_pages, const int32_t* page_table,
                     void* summaries, const int32_t* seq_lens, float* out, int32_t* selected,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The three steps of se_sparse_decode, exposed one by one. */

/* scores: fp32 [B, Hkv, max_pages_per_seq]; entries past a request's pages
 * are not written; for a request that runs dense only the summary refresh
 * happens. */
int se_quest_scores(const se_kv_layout* layout, const se_decode_params* params, const void* q,
                    const void* k_pages, const int32_t* page_table, void* summaries,
                    const int32_t* seq_lens, float* scores, void* stream);

/* selected: int32 [B, Hkv, kcap] from scores laid out as above (scores are
 * not read when topk = 0). */
int se_topk_pages(const se_decode_params* params, int32_t num_kv_heads, const float* scores,
                  const int32_t* seq_lens, int32_t* selected, void* stream);

/* Attention over the pages listed in `selected` ([B, Hkv, kcap], ascending,
 * -1 padded), or over every page of each request when `selected` is NULL.
 * workspace as for se_sparse_decode. */
int se_decode_selected(const se_kv_layout* layout, const se_decode_params* params, const void* q,
                       const void* k_pages, const void* v_pages, const int32_t* page_table,
                       const int32_t* seq_lens, const int32_t* selected, float* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * For callers that cannot allocate or pass a workspace: code under HIP graph
 * capture that may not call hipMalloc, tight serving loops, harnesses that
 * forbid allocation.
 *
 * se_sparse_decode_noalloc is se_sparse_decode (same arguments, same
 * kernels, same results) with its workspace in a device array that the
 * library holds: SE_NOALLOC_SCRATCH_BYTES on each GPU the call runs on, kept
 * until the process ends.  It allocates nothing and calls no allocating
 * routine.  The first call on a GPU looks the array's address up (that GPU
 * must be the current device) and keeps it.
 *   - The step must fit the array: se_sparse_decode_workspace_size of the
 *     same layout and params must not exceed SE_NOALLOC_SCRATCH_BYTES, else
 *     SE_EWORKSPACE.  (Batch 8 at 32K tokens with 8 KV heads takes 1.6 MiB,
 *     batch 32 at 128K with 4 KV heads 20.5 MiB, 16 latent-attention
 *     requests of up to 128K tokens 16.6 MiB.)
 *   - `stream` must belong to the current device (SE_EINVAL otherwise);
 *     SE_EHIP if the array's address cannot be obtained.
 *   - Every call on one GPU uses the same array, and the array keeps what the
 *     last call left (no call needs it cleared).  Calls that may overlap on
 *     one GPU -- different streams without ordering between them -- race on
 *     it: the caller must order them.
 * ------------------------------------------------------------------------- */
#define SE_NOALLOC_SCRATCH_BYTES (32u << 20)

int se_sparse_decode_noalloc(const se_kv_layout* layout, const se_decode_params* params, const void* q,
                             const void* k_pages, const void* v_pages, const int32_t* page_table, void* summaries,
                             const int32_t* seq_lens, float* out, int32_t* selected, void* stream);

/* ---------------------------------------------------------------------------
 * SnapKV eviction and compaction, and the eviction family around it.
 *
 * Per request b (prompt length n = prompt_lens[b]) and KV head g, with
 * L = n - window:
 *   - window row i (absolute position L+i) of each query head h of g has
 *     logits z_j = s * q_win[b][h][i] . k[b][g][j] over its causal history
 *     j <= L+i, normalised by a softmax over that history;
 *   - votes S_j = sum over the group's heads and window rows of those
 *     probabilities, for prefix positions j < L;
 *   - pooled votes = stride-1 centred max-pool of odd width pool_kernel,
 *     cut at both ends of the prefix;
 *   - candidates [lo, hi): lo = max(sink, interval_begin),
 *     hi = min(n - max(recent, window), interval_end) (interval_end = n when
 *     no interval is given); every position outside them is kept;
 *   - kept = 0..lo-1, the `budget` candidates with the largest pooled vote
 *     (ties to the lower position), and hi..n-1, in ascending order; when
 *     hi - lo <= budget every position 0..n-1 is kept.  With sink = recent
 *     = 0 and no interval this is SnapKV's top-R prefix plus the window;
 *   - k_out[b][g][r] = k[b][g][kept[r]] and likewise v_out (bit copies).
 *
 * The methods of the pages' tables as settings of these fields:
 *   SnapKV (Table 8)     window 32, pool 7, budget 2016, recent 32
 *   SnapKV (Table 9)     window 16, pool 7, budget 4096, sink 16, recent 64
 *   H2O (Table 8)        window 128, pool 1, total T = 8192 split by the
 *                        recent ratio 0.5: recent = 4096, budget = 4096
 *   PyramidKV (Table 8)  window 32, sink 64, recent 512, budget per layer
 *                        from se_pyramid_budgets(L, 4096, 0.6, 0.01)
 *   prefix-cache pruning an interval [ib, ie) naming the history span that
 *   (Figure 4)           may be pruned; everything outside it is kept
 * ------------------------------------------------------------------------- */
typedef struct se_snapkv_params {
  int32_t batch;           /* B                                              */
  int32_t num_q_heads;     /* Hq, a multiple of num_kv_heads, G <= 32         */
  int32_t num_kv_heads;    /* Hkv                                            */
  int32_t head_dim;        /* D; 128 or 64                                   */
  int32_t max_prompt_len;  /* token dim of k, v: [B, Hkv, max_prompt_len, D];
                              max_prompt_len - window <= 65536 (longer:
                              SE_EUNSUPPORTED)                             */
  int32_t window;          /* W, 1..128                                       */
  int32_t pool_kernel;     /* odd, 1 .. 129 (wider: SE_EUNSUPPORTED)          */
  int32_t budget;          /* R >= 1 candidates kept                          */
  int32_t out_capacity;    /* token dim of k_out/v_out, >= the kept capacity  */
  float sm_scale;          /* s; 0 means 1/sqrt(D)                            */
  int32_t sink;            /* >= 0 leading positions always kept              */
  int32_t recent;          /* >= 0 trailing positions always kept (at least
                              the window is)                                 */
  int32_t interval_begin;  /* history interval [begin, end) that may be      */
  int32_t interval_end;    /* pruned, 0 <= begin < end <= max_prompt_len;
                              both 0: no interval                            */
} se_snapkv_params;

/* Row length kcap of kept_idx: the most positions a request of any length up
 * to max_prompt_len keeps, max(sink, interval_begin) + budget +
 * max(recent, window, max_prompt_len - interval_end); budget + window for
 * plain SnapKV.  out_capacity must be at least kcap. */
int se_snapkv_kept_capacity(const se_snapkv_params* params, int32_t* kcap);

int se_snapkv_workspace_size(const se_snapkv_params* params, size_t* bytes);

/*   q_win       bf16 [B, Hq, W, D]   queries of the last W prompt positions
 *   k, v        bf16 [B, Hkv, max_prompt_len, D]
 *   prompt_lens int32 [B], each in [1, max_prompt_len]
 *   k_out,v_out bf16 [B, Hkv, out_capacity, D]; rows past kept_len untouched;
 *               must not overlap k or v (SE_EINVAL)
 *   kept_idx    int32 [B, Hkv, kcap], ascending, -1 padded
 *   kept_len    int32 [B, Hkv]
 * After the call completes the caller may release k and v. */
int se_snapkv_compact(const se_snapkv_params* params, const void* q_win, const void* k, const void* v,
                      const int32_t* prompt_lens, void* k_out, void* v_out, int32_t* kept_idx,
                      int32_t* kept_len, void* workspace, size_t workspace_bytes, void* stream);

/* Re-eviction of a cache that was compacted before (SparseEngine Tables 9-10:
 * SnapKV, H2O and PyramidKV evict again every 1,024 decode steps).  k, v are
 * the retained cache [B, Hkv, max_prompt_len, D] with the decode steps'
 * rows appended; cache_lens[b] counts its rows (kept prompt rows plus decode
 * steps); q_win holds the queries of the last W decode steps.  Everything is
 * computed as in se_snapkv_compact over the rows of the cache, except that
 * kept_idx receives original positions: positions int32 [B, Hkv,
 * max_prompt_len] gives the position row r of (b, g) stands for (the
 * previous kept_idx, followed by the decode steps' positions).  positions
 * must be non-NULL when batch > 0 (SE_EINVAL); k_out/v_out must not overlap
 * k/v (the caller double-buffers). */
int se_snapkv_recompact(const se_snapkv_params* params, const void* q_win, const void* k, const void* v,
                        const int32_t* cache_lens, const int32_t* positions, void* k_out, void* v_out,
                        int32_t* kept_idx, int32_t* kept_len, void* workspace, size_t workspace_bytes,
                        void* stream);

/* PyramidKV's selected budget per layer (SparseEngine Tables 8-9: "layer
 * ratios 0.6 to 0.01 (linear)"; Table 11: 0.6 to 0.0154712 from layer 0).
 * HOST function, no GPU work: budgets is a HOST array [num_layers].  Layer
 * l's budget is proportional to r_l = ratio_first + (ratio_last -
 * ratio_first) * l / (num_layers - 1); the layers share num_layers * budget
 * tokens, dealt as the floors of the exact shares plus one token each to
 * the layers with the largest remainders (ties to the lower layer).  Ratios
 * are taken to nine decimals (rounded half to even) and the shares are exact
 * integer arithmetic.  Errors: SE_EINVAL for a NULL array, num_layers < 1,
 * budget < 1 or a ratio outside (0, 1000]; SE_EUNSUPPORTED for more than
 * 4096 layers or a budget above 2^24.  A layer's budget can be 0 for a
 * vanishing ratio; callers evict with budget >= 1. */
int se_pyramid_budgets(int32_t num_layers, int32_t budget, double ratio_first, double ratio_last,
                       int32_t* budgets);

/* The steps of se_snapkv_compact, exposed one by one.
 * votes/pooled: fp32 [B, Hkv, max_prompt_len]; entries j < L are written for
 * every request with n > W (se_snapkv_votes) and n - W > budget is not
 * required; other entries are untouched.  se_snapkv_votes needs the same
 * workspace as se_snapkv_compact.  se_maxpool1d pools the whole prefix;
 * se_snapkv_select writes kept_idx [B, Hkv, kcap] of prompt positions and
 * se_compact copies the rows kept_idx names (k_out/v_out must not overlap
 * k/v: SE_EINVAL). */
int se_snapkv_votes(const se_snapkv_params* params, const void* q_win, const void* k,
                    const int32_t* prompt_lens, float* votes, void* workspace, size_t workspace_bytes,
                    void* stream);
int se_maxpool1d(const se_snapkv_params* params, const float* votes, const int32_t* prompt_lens,
                 float* pooled, void* stream);
int se_snapkv_select(const se_snapkv_params* params, const float* pooled, const int32_t* prompt_lens,
                     int32_t* kept_idx, int32_t* kept_len, void* stream);
int se_compact(const se_snapkv_params* params, const void* k, const void* v, const int32_t* kept_idx,
               const int32_t* kept_len, void* k_out, void* v_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_KV_SE_H_ */
