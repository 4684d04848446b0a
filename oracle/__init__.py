"""Plain fp64 CPU oracle for Quest sparse decode and SnapKV eviction.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The library (``sparse_kv_long_amd``) never does, and this package
never imports the library: the two share no code.

The oracle is written from the SparseEngine pages (arXiv 2609.39068) and the
plain reading of the problem they pose.  It is slow on purpose: numpy fp64,
one (request, KV head) unit at a time, with only a matmul or a sort from the
library as a step.  Inputs arrive as raw bf16 bit patterns (``uint16``) and
are decoded exactly (bf16 -> fp32 by a 16-bit shift -> fp64).

What is computed, step by step (names follow the pages' notation where they
give one: prompt length n, key position j, logit z, weight alpha -- appendix
Table 7):

  O1  page summaries: per page and KV head, channel-wise min and max of the
      keys of the page's valid tokens (Fig. 3 caption: radix prefix caching
      "attaches the summaries required by Quest"; Table 8: 16-token pages).
  O2  page bound: U = s * sum_c max(q_c * min_c, q_c * max_c), an upper bound
      of s * q.k over the page's keys.
  O3  KV-head score: max of U over the query heads that share the KV head.
  O4  selection: the min(topk, pages) pages with the largest score, ties to
      the lower page id, returned ascending; optionally with always-kept sink
      and recent pages beside the selected budget (appendix Tables 8-11).
  O5  attention: softmax attention of each query head over the valid tokens
      of its KV head's selected pages (Table 7: logit z, weight alpha).
  O6  SnapKV: window-row softmax over each row's causal history (Table 7:
      "[i]" includes the current token), votes summed over the group's heads
      and window rows for the prefix columns, 1-D max-pool (Table 8: 32
      scoring window, pooling kernel 7), top-R retain plus the window,
      compaction by copying the kept rows (Table 15 note: physical eviction
      releases storage).
  O7  decode over the compacted cache: O5 with every kept row selected.
  O8  the eviction family around O6's scores (appendix Tables 8-11): always
      kept sink and recent tokens beside the selected budget (SnapKV rows
      with a Sink and a Recent column; H2O's recent ratio with its 128-token
      scoring window), a history interval outside which nothing is evicted
      (Figure 4: prefix-cache pruning), and re-eviction of an already
      compacted cache whose rows carry their original positions (Tables 9-10:
      "eviction every 1,024 decode steps").
  O9  PyramidKV's per-layer budgets: layer ratios falling linearly from the
      first to the last layer (Tables 8-9, 11).

Readings where the pages are silent are listed in the design notes; the ones
that change numbers are noted next to the code that takes them.

Parity status: every function here is pinned by a test in
``tests/test_oracle_*.py`` (worked examples, brute force, closed forms and
invariants); none is "parity unpinned" except the input generators in
``synth`` (a definition, not a result).
"""
from __future__ import annotations

import math

import numpy as np

PAGE = 16


# ----------------------------------------------------------------------------
# bf16 decoding
# ----------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: the top 16 bits of an IEEE fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def pages_of(n: int, page_size: int = PAGE) -> int:
    """Number of pages that hold n tokens."""
    return (int(n) + page_size - 1) // page_size


# ----------------------------------------------------------------------------
# Per-unit steps (one request b, one KV head g)
# ----------------------------------------------------------------------------
def gather_unit_pages(pages_bits, page_table_row, g: int, n: int, page_size: int = PAGE) -> np.ndarray:
    """Logical pages 0..P_b-1 of one (request, KV head) as fp64 [P_b, page_size, D].

    Slots past the n valid tokens are returned as NaN so that any later use of
    them poisons the result instead of passing silently.
    """
    P = pages_of(n, page_size)
    phys = np.asarray(page_table_row[:P], dtype=np.int64)
    x = bf16_to_f64(np.asarray(pages_bits)[phys, g])  # [P, ps, D]
    x = x.copy()
    tail = n - (P - 1) * page_size if P else 0
    if P and tail < page_size:
        x[P - 1, tail:, :] = np.nan
    return x


def unit_summaries(keys_pages: np.ndarray, n: int, page_size: int = PAGE):
    """O1: channel-wise (min, max) of the valid keys of each page: 2 x [P_b, D]."""
    P, ps, D = keys_pages.shape
    mins = np.empty((P, D))
    maxs = np.empty((P, D))
    for p in range(P):
        valid = min(ps, n - p * page_size)
        rows = keys_pages[p, :valid, :]
        mins[p] = rows.min(axis=0)
        maxs[p] = rows.max(axis=0)
    return mins, maxs


def unit_page_bounds(q_heads: np.ndarray, mins: np.ndarray, maxs: np.ndarray, scale: float) -> np.ndarray:
    """O2: U[h, p] = s * sum_c max(q[h,c] * min[p,c], q[h,c] * max[p,c]).

    For every key k in page p, q.k <= U/s channel by channel, because each
    k_c lies in [min_c, max_c] and q_c * k_c is linear in k_c.
    """
    a = q_heads[:, None, :] * mins[None, :, :]
    b = q_heads[:, None, :] * maxs[None, :, :]
    return float(scale) * np.maximum(a, b).sum(axis=2)


def unit_kv_head_score(U: np.ndarray, mode: str = "max") -> np.ndarray:
    """O3: one score per page for the KV head, from its query heads' bounds.

    Reading: the max over the group keeps the upper-bound meaning at KV-head
    level ("sum" is the alternative reading, kept as a switch).
    """
    if mode == "max":
        return U.max(axis=0)
    if mode == "sum":
        return U.sum(axis=0)
    raise ValueError(mode)


def unit_select(scores: np.ndarray, topk: int) -> np.ndarray:
    """O4: the min(topk, P) ids with the largest score, ties to the lower id, ascending."""
    P = len(scores)
    k = min(int(topk), P)
    order = sorted(range(P), key=lambda p: (-float(scores[p]), p))
    return np.array(sorted(order[:k]), dtype=np.int64)


def unit_select_forced(scores: np.ndarray, topk: int, sink: int, recent: int) -> np.ndarray:
    """O4 with always-kept pages: the first ``sink`` and the last ``recent``
    pages of the request, plus the ``topk`` pages of largest score among the
    others (ties to the lower id), ascending.

    SparseEngine appendix Tables 8-11 list a Sink and a Recent budget beside
    each method's selected budget, and Table 10's caption says the selected
    budget excludes them (Quest there: 64 sink + 512 recent + 1,472 selected
    = 2,048 tokens); the StreamingLLM rows have sink and recent only, which is
    topk = 0 here.  Budgets are in pages (16 tokens each).
    """
    P = len(scores)
    forced = set(range(min(int(sink), P))) | set(range(max(P - int(recent), 0), P))
    rest = [p for p in range(P) if p not in forced]
    ranked = sorted(rest, key=lambda p: (-float(scores[p]), p))
    chosen = forced | set(ranked[:max(int(topk), 0)])
    return np.array(sorted(chosen), dtype=np.int64)


def unit_attention(q_heads: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float) -> np.ndarray:
    """O5: out[h] = sum_t alpha[h,t] v_t with alpha = softmax_t(s * q_h . k_t).

    The max is subtracted before exponentiating; an empty token set gives 0.
    """
    G = q_heads.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((G, vals.shape[1]))
    z = float(scale) * (q_heads @ keys.T)  # [G, T]
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    alpha = w / w.sum(axis=1, keepdims=True)
    return alpha @ vals


def unit_selected_tokens(pages: np.ndarray, sel: np.ndarray, n: int, page_size: int = PAGE) -> np.ndarray:
    """Rows of the valid tokens of the selected pages, in page order: [T, D]."""
    rows = []
    for p in sel:
        valid = min(page_size, n - int(p) * page_size)
        rows.append(pages[int(p), :valid, :])
    if not rows:
        return np.zeros((0, pages.shape[2]))
    return np.concatenate(rows, axis=0)


# ----------------------------------------------------------------------------
# Split-K partials and their merge (log-sum-exp)
# ----------------------------------------------------------------------------
def attention_partial(q_heads, keys, vals, scale):
    """Unnormalised partial over a token subset: (m [G], l [G], acc [G, Dv])."""
    G = q_heads.shape[0]
    if keys.shape[0] == 0:
        return np.full(G, -np.inf), np.zeros(G), np.zeros((G, vals.shape[1]))
    z = float(scale) * (q_heads @ keys.T)
    m = z.max(axis=1)
    w = np.exp(z - m[:, None])
    return m, w.sum(axis=1), w @ vals


def merge_partials(parts):
    """out = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s with M = max_s m_s."""
    ms = np.stack([p[0] for p in parts])  # [S, G]
    M = ms.max(axis=0)
    Msafe = np.where(np.isfinite(M), M, 0.0)
    num = 0.0
    den = 0.0
    for m, l, acc in parts:
        f = np.where(np.isfinite(m), np.exp(m - Msafe), 0.0)
        num = num + f[:, None] * acc
        den = den + f * l
    den = np.where(den > 0, den, 1.0)
    return num / den[:, None]


# ----------------------------------------------------------------------------
# Batch wrappers for the Quest decode step
# ----------------------------------------------------------------------------
def quest_summaries(k_pages, page_table, seq_lens, page_size: int = PAGE):
    """O1 for every request and KV head: fp64 [B, max_pages, Hkv, 2, D], NaN past P_b."""
    k_pages = np.asarray(k_pages)
    B, MP = np.asarray(page_table).shape
    Hkv, D = k_pages.shape[1], k_pages.shape[3]
    out = np.full((B, MP, Hkv, 2, D), np.nan)
    for b in range(B):
        n = int(seq_lens[b])
        for g in range(Hkv):
            kp = gather_unit_pages(k_pages, page_table[b], g, n, page_size)
            mn, mx = unit_summaries(kp, n, page_size)
            P = mn.shape[0]
            out[b, :P, g, 0] = mn
            out[b, :P, g, 1] = mx
    return out


def quest_scores(q, summaries, seq_lens, group: int, scale: float, page_size: int = PAGE,
                 mode: str = "max"):
    """O2+O3: KV-head page scores [B, Hkv, max_pages] (-inf past P_b).

    ``summaries`` is the fp64 [B, max_pages, Hkv, 2, D] array of O1.
    """
    qf = bf16_to_f64(q)
    B, MP, Hkv = summaries.shape[:3]
    A = np.full((B, Hkv, MP), -np.inf)
    for b in range(B):
        P = pages_of(seq_lens[b], page_size)
        for g in range(Hkv):
            U = unit_page_bounds(qf[b, g * group:(g + 1) * group], summaries[b, :P, g, 0],
                                 summaries[b, :P, g, 1], scale)
            A[b, g, :P] = unit_kv_head_score(U, mode)
    return A


def quest_select(A, seq_lens, topk: int, page_size: int = PAGE, sink: int = 0, recent: int = 0):
    """O4 for every (request, KV head): nested list of ascending id arrays
    (with always-kept sink and recent pages when either is non-zero)."""
    B, Hkv, _ = A.shape
    out = []
    for b in range(B):
        P = pages_of(seq_lens[b], page_size)
        if sink or recent:
            out.append([unit_select_forced(A[b, g, :P], topk, sink, recent) for g in range(Hkv)])
        else:
            out.append([unit_select(A[b, g, :P], topk) for g in range(Hkv)])
    return out


def sparse_attention(q, k_pages, v_pages, page_table, seq_lens, selection, group: int, scale: float,
                     head_dim_v: int, v_is_k_prefix: bool = False, page_size: int = PAGE):
    """O5 for the whole batch, over a given selection: out fp64 [B, Hq, Dv]."""
    qf = bf16_to_f64(q)
    B, Hq, _ = qf.shape
    Hkv = Hq // group
    out = np.zeros((B, Hq, head_dim_v))
    for b in range(B):
        n = int(seq_lens[b])
        for g in range(Hkv):
            kp = gather_unit_pages(k_pages, page_table[b], g, n, page_size)
            if v_is_k_prefix:
                vp = kp[..., :head_dim_v]
            else:
                vp = gather_unit_pages(v_pages, page_table[b], g, n, page_size)
            sel = np.asarray(selection[b][g], dtype=np.int64)
            keys = unit_selected_tokens(kp, sel, n, page_size)
            vals = unit_selected_tokens(vp, sel, n, page_size)
            out[b, g * group:(g + 1) * group] = unit_attention(qf[b, g * group:(g + 1) * group], keys, vals, scale)
    return out


def sparse_decode(q, k_pages, v_pages, page_table, seq_lens, topk: int, group: int, scale: float,
                  head_dim_v: int, v_is_k_prefix: bool = False, page_size: int = PAGE, mode: str = "max",
                  sink: int = 0, recent: int = 0):
    """The whole Quest decode step O1-O5.  Returns (out, selection, scores)."""
    summ = quest_summaries(k_pages, page_table, seq_lens, page_size)
    A = quest_scores(q, summ, seq_lens, group, scale, page_size, mode)
    sel = quest_select(A, seq_lens, topk, page_size, sink, recent)
    out = sparse_attention(q, k_pages, v_pages, page_table, seq_lens, sel, group, scale, head_dim_v,
                           v_is_k_prefix, page_size)
    return out, sel, A


def dense_attention(q, keys, vals, group: int, scale: float):
    """Plain GQA softmax attention: q [Hq, Dk], keys [Hkv, T, Dk], vals [Hkv, T, Dv] (fp64)."""
    Hq = q.shape[0]
    out = np.zeros((Hq, vals.shape[2]))
    for g in range(keys.shape[0]):
        out[g * group:(g + 1) * group] = unit_attention(q[g * group:(g + 1) * group], keys[g], vals[g], scale)
    return out


# ----------------------------------------------------------------------------
# SnapKV (O6) and decode over the compacted cache (O7)
# ----------------------------------------------------------------------------
def snapkv_unit_votes(q_win: np.ndarray, keys: np.ndarray, n: int, scale: float):
    """Votes of one (request, KV head).

    q_win: fp64 [G, W, D], the last W queries of each head of the group, row i
    at absolute position n-W+i.  keys: fp64 [>=n, D].  Row i's logits are
    z_j = s q_i . k_j over its causal history j <= n-W+i (the current token
    included, appendix Table 7), normalised by a softmax over that history.
    Returns (S [n-W], row_max [G, W], row_sum [G, W]): S_j sums the
    probabilities of prefix column j < n-W over all heads and rows.
    """
    G, W, D = q_win.shape
    L = n - W
    K = keys[:n]
    Q = q_win.reshape(G * W, D)
    z = float(scale) * (Q @ K.T)  # [G*W, n]
    rows_pos = L + np.tile(np.arange(W), G)  # absolute position of each row
    cols = np.arange(n)
    z = np.where(cols[None, :] <= rows_pos[:, None], z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    P = e / l
    S = P[:, :L].sum(axis=0)
    return S, m.reshape(G, W), l.reshape(G, W)


def maxpool1d(S: np.ndarray, kernel: int) -> np.ndarray:
    """Stride-1 centred max-pool of odd width; the window is cut at both ends."""
    r = kernel // 2
    L = len(S)
    out = np.empty(L)
    for j in range(L):
        out[j] = S[max(0, j - r):min(L, j + r + 1)].max()
    return out


def snapkv_unit_keep(pooled: np.ndarray, n: int, window: int, budget: int) -> np.ndarray:
    """Kept positions, ascending: the top-``budget`` prefix positions by pooled
    vote (ties to the lower position) plus the whole window; everything when
    the prefix already fits the budget."""
    L = n - window
    if L <= budget:
        return np.arange(n, dtype=np.int64)
    top = unit_select(pooled, budget)
    return np.concatenate([top, np.arange(L, n, dtype=np.int64)])


def eviction_candidates(n: int, window: int, sink: int = 0, recent: int = 0, interval=None):
    """O8: the range [lo, hi) of positions an eviction may drop; every
    position outside it is kept.

    The first ``sink`` positions are kept, and so are the last
    max(recent, window) positions: the scoring window is always part of the
    recent tokens (SnapKV keeps its window; appendix Tables 8-11 give each
    method a Sink and a Recent budget beside the selected one, and H2O's
    recent ratio reserves a share of its budget for the newest tokens).  With
    a history interval [ib, ie) (Figure 4: the application names the span
    that may be pruned) the range is further cut to it.  hi <= lo means there
    is nothing to choose from.
    """
    lo = int(sink)
    hi = int(n) - max(int(recent), int(window))
    if interval is not None:
        lo = max(lo, int(interval[0]))
        hi = min(hi, int(interval[1]))
    return lo, hi


def eviction_unit_keep(pooled: np.ndarray, n: int, window: int, budget: int, sink: int = 0, recent: int = 0,
                       interval=None) -> np.ndarray:
    """O8: kept positions, ascending.  Everything outside the candidate range
    [lo, hi) is kept; inside it the ``budget`` positions with the largest
    pooled vote (ties to the lower position); when the range holds no more
    than ``budget`` positions nothing is dropped.  ``pooled`` covers the
    scored prefix [0, n - window).  With sink = recent = 0 and no interval
    this is O6's selection (top budget of the prefix plus the window)."""
    lo, hi = eviction_candidates(n, window, sink, recent, interval)
    if hi - lo <= budget:
        return np.arange(n, dtype=np.int64)
    top = lo + unit_select(np.asarray(pooled)[lo:hi], budget)
    return np.concatenate([np.arange(lo, dtype=np.int64), top, np.arange(hi, n, dtype=np.int64)])


def eviction_kept_capacity(max_len: int, window: int, budget: int, sink: int = 0, recent: int = 0,
                           interval=None) -> int:
    """The most positions O8 can keep for any prompt length up to ``max_len``:
    max(sink, ib) + budget + max(recent, window, max_len - ie).  A kept list
    is at most this long whether or not anything is dropped."""
    ib, ie = (0, int(max_len)) if interval is None else (int(interval[0]), int(interval[1]))
    return max(int(sink), ib) + int(budget) + max(int(recent), int(window), int(max_len) - ie)


def snapkv_compact(q_win, k, v, prompt_lens, group: int, scale: float, window: int, pool_kernel: int,
                   budget: int, out_capacity: int, sink: int = 0, recent: int = 0, interval=None,
                   positions=None):
    """O6 (with O8's forced positions and interval) for the whole batch.

    q_win bf16 bits [B, Hq, W, D]; k, v bf16 bits [B, Hkv, Nmax, D].
    Returns (k_out, v_out, kept_idx, kept_len, pooled) where k_out/v_out are
    bf16 bit arrays [B, Hkv, out_capacity, D] holding the kept rows (rows past
    kept_len are zero), kept_idx is int [B, Hkv, kcap] padded with -1 (kcap =
    eviction_kept_capacity; budget + window without forced positions or an
    interval), and pooled[b][g] is the pooled vote vector over the prefix
    (None when nothing is scored).

    ``positions`` (int [B, Hkv, Nmax], optional) re-evicts a cache that was
    compacted before: row r of k/v holds the token at original position
    positions[b][g][r], and kept_idx reports those original positions (the
    rows copied are still the kept rows of k/v).  Nothing else changes: the
    window is the last W rows of the cache and the softmax runs over its rows.
    """
    qf = bf16_to_f64(q_win)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hkv, Nmax, D = k.shape
    cap = eviction_kept_capacity(Nmax, window, budget, sink, recent, interval)
    k_out = np.zeros((B, Hkv, out_capacity, D), dtype=np.uint16)
    v_out = np.zeros((B, Hkv, out_capacity, D), dtype=np.uint16)
    kept_idx = np.full((B, Hkv, cap), -1, dtype=np.int64)
    kept_len = np.zeros((B, Hkv), dtype=np.int64)
    pooled = [[None] * Hkv for _ in range(B)]
    for b in range(B):
        n = int(prompt_lens[b])
        lo, hi = eviction_candidates(n, window, sink, recent, interval)
        for g in range(Hkv):
            if hi - lo <= budget:
                keep = np.arange(n, dtype=np.int64)
            else:
                keys = bf16_to_f64(k[b, g, :n])
                S, _, _ = snapkv_unit_votes(qf[b, g * group:(g + 1) * group], keys, n, scale)
                Sp = maxpool1d(S, pool_kernel)
                pooled[b][g] = Sp
                keep = eviction_unit_keep(Sp, n, window, budget, sink, recent, interval)
            kept_len[b, g] = len(keep)
            kept_idx[b, g, :len(keep)] = keep if positions is None else np.asarray(positions)[b, g, keep]
            k_out[b, g, :len(keep)] = k[b, g, keep]
            v_out[b, g, :len(keep)] = v[b, g, keep]
    return k_out, v_out, kept_idx, kept_len, pooled


def pyramid_budgets(num_layers: int, budget: int, ratio_first: float, ratio_last: float):
    """O9: PyramidKV's selected budget per layer.

    The pages give layer ratios falling linearly from the first layer to the
    last (Tables 8-9: 0.6 to 0.01; Table 11: 0.6 to 0.0154712 from layer 0)
    beside one selected budget.  Reading: layer l's budget is proportional to
    its ratio r_l = ratio_first + (ratio_last - ratio_first) * l / (L - 1),
    and the layers share L * budget tokens in all, so the budgets average the
    configured one.  The ratios are taken to nine decimals and the shares are
    computed exactly (integers); the L * budget tokens are dealt as the
    floors of the exact shares plus one more token to each of the layers with
    the largest remainders, ties to the lower layer.
    """
    L = int(num_layers)
    A = round(float(ratio_first) * 10**9)
    Z = round(float(ratio_last) * 10**9)
    if L == 1:
        weights = [A]
    else:
        weights = [A * (L - 1) + (Z - A) * l for l in range(L)]  # r_l scaled by 1e9 * (L - 1)
    total_w = sum(weights)
    tokens = L * int(budget)
    share = [tokens * w for w in weights]  # layer l's exact share is share[l] / total_w
    floors = [s // total_w for s in share]
    rems = [s % total_w for s in share]
    extra = tokens - sum(floors)
    order = sorted(range(L), key=lambda l: (-rems[l], l))
    out = list(floors)
    for l in order[:extra]:
        out[l] += 1
    return out


def decode_over_rows(q, keys_bits, vals_bits, length: int, group: int, scale: float):
    """O7: one decode step over the first ``length`` rows of a dense per-head cache.

    q bf16 bits [Hq, D]; keys/vals bf16 bits [Hkv, >=length, D].
    """
    return dense_attention(bf16_to_f64(q), bf16_to_f64(np.asarray(keys_bits)[:, :length]),
                           bf16_to_f64(np.asarray(vals_bits)[:, :length]), group, scale)
