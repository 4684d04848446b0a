"""The oracle's pins catch plausible mistakes.

Each case below plants one mistake in a copy of an oracle step (a wrong sign,
a dropped term, a missing scale, an off-by-one mask, a wrong tie order, a
transposed pairing, ...) and runs every pin of the oracle against it on the
CPU; at least one pin must fail.  Nothing here touches the GPU path.
"""
from unittest import mock

import numpy as np
import pytest

import oracle
import test_oracle_eviction as te
import test_oracle_quest as tq
import test_oracle_snapkv as ts

PAGE = oracle.PAGE


def _pins():
    """Every oracle pin, with fixed examples for the property-based ones."""
    return [
        tq.test_worked_example_w1,
        tq.test_summaries_brute_force,
        lambda: tq.test_bound_is_an_upper_bound_of_every_logit.hypothesis.inner_test(seed=3, D=8, G=2, n=37,
                                                                                      scale=0.7),
        lambda: tq.test_bound_is_an_upper_bound_of_every_logit.hypothesis.inner_test(seed=4, D=64, G=4, n=200,
                                                                                      scale=0.09),
        tq.test_bound_tight_on_single_key_pages_and_zero_query,
        tq.test_kv_head_score_is_max_over_group,
        lambda: tq.test_selection_against_pairwise_order.hypothesis.inner_test(seed=5, P=40, topk=9, levels=3),
        lambda: tq.test_selection_against_pairwise_order.hypothesis.inner_test(seed=6, P=17, topk=30, levels=2),
        lambda: tq.test_dense_case_equals_library_attention(4, 64, (100, 1)),
        tq.test_forced_selection_special_cases,
        lambda: tq.test_forced_selection_against_its_definition.hypothesis.inner_test(seed=12, P=23, topk=4, sink=2,
                                                                                      recent=3, levels=3),
        tq.test_sparse_output_is_convex_combination_of_selected_rows,
        tq.test_split_merge_equals_single_softmax,
        ts.test_worked_example_w2,
        lambda: ts.test_votes_brute_force_and_mass.hypothesis.inner_test(seed=7, G=2, W=3, L=12, D=3, s=0.8),
        lambda: ts.test_maxpool_properties.hypothesis.inner_test(seed=8, L=25, kern=7),
        lambda: ts.test_maxpool_properties.hypothesis.inner_test(seed=9, L=6, kern=1),
        ts.test_identity_budget_keeps_everything_bitwise,
        ts.test_eviction_keeps_top_pooled_plus_window,
        ts.test_decode_over_compacted_cache,
        te.test_worked_example_w3,
        lambda: te.test_selection_against_pairwise_order.hypothesis.inner_test(
            seed=13, n=40, W=3, R=6, sink=2, recent=7, use_iv=False, ib=0, span=1, levels=3),
        lambda: te.test_selection_against_pairwise_order.hypothesis.inner_test(
            seed=14, n=50, W=2, R=4, sink=0, recent=0, use_iv=True, ib=10, span=20, levels=50),
        lambda: te.test_defaults_reduce_to_snapkv.hypothesis.inner_test(seed=15, n=30, W=3, R=5),
        te.test_compact_with_forced_positions_and_interval,
        te.test_reeviction_reports_original_positions,
        te.test_pyramid_worked_examples,
        lambda: te.test_pyramid_exact_shares.hypothesis.inner_test(L=47, R=4096, a=0.6, z=0.01),
        te.test_pyramid_special_cases,
    ]


# --- planted mistakes: each is a wrong variant of one oracle step -------------
def bound_min_instead_of_max(q, mins, maxs, scale):
    return float(scale) * np.minimum(q[:, None, :] * mins[None], q[:, None, :] * maxs[None]).sum(axis=2)


def bound_max_term_only(q, mins, maxs, scale):
    return float(scale) * (q[:, None, :] * maxs[None]).sum(axis=2)


def bound_without_scale(q, mins, maxs, scale):
    return np.maximum(q[:, None, :] * mins[None], q[:, None, :] * maxs[None]).sum(axis=2)


def bound_split_sign_swapped(q, mins, maxs, scale):
    qp, qn = np.maximum(q, 0), np.minimum(q, 0)
    return float(scale) * (qp @ mins.T + qn @ maxs.T)


def head_score_sum(U, mode="max"):
    return U.sum(axis=0)


def head_score_mean(U, mode="max"):
    return U.mean(axis=0)


def select_ties_to_higher_id(scores, topk):
    P = len(scores)
    order = sorted(range(P), key=lambda p: (-float(scores[p]), -p))
    return np.array(sorted(order[:min(topk, P)]), dtype=np.int64)


def select_in_score_order(scores, topk):
    P = len(scores)
    order = sorted(range(P), key=lambda p: (-float(scores[p]), p))
    return np.array(order[:min(topk, P)], dtype=np.int64)


def select_one_short(scores, topk):
    P = len(scores)
    order = sorted(range(P), key=lambda p: (-float(scores[p]), p))
    return np.array(sorted(order[:max(min(topk, P) - 1, 0)]), dtype=np.int64)


def forced_inside_budget(scores, topk, sink, recent):
    P = len(scores)
    forced = set(range(min(sink, P))) | set(range(max(P - recent, 0), P))
    rest = sorted((p for p in range(P) if p not in forced), key=lambda p: (-float(scores[p]), p))
    return np.array(sorted(forced | set(rest[:max(topk - len(forced), 0)])), dtype=np.int64)


def forced_recent_one_short(scores, topk, sink, recent):
    P = len(scores)
    forced = set(range(min(sink, P))) | set(range(max(P - recent + 1, 0), P))
    rest = sorted((p for p in range(P) if p not in forced), key=lambda p: (-float(scores[p]), p))
    return np.array(sorted(forced | set(rest[:topk])), dtype=np.int64)


def summaries_over_whole_last_page(keys_pages, n, page_size=PAGE):
    return keys_pages.min(axis=1), keys_pages.max(axis=1)


def summaries_drop_last_valid_token(keys_pages, n, page_size=PAGE):
    P, ps, D = keys_pages.shape
    mins, maxs = np.empty((P, D)), np.empty((P, D))
    for p in range(P):
        valid = max(1, min(ps, n - p * page_size) - 1)
        mins[p] = keys_pages[p, :valid].min(axis=0)
        maxs[p] = keys_pages[p, :valid].max(axis=0)
    return mins, maxs


def attention_without_scale(q, keys, vals, scale):
    if keys.shape[0] == 0:
        return np.zeros((q.shape[0], vals.shape[1]))
    z = q @ keys.T
    w = np.exp(z - z.max(axis=1, keepdims=True))
    return (w / w.sum(axis=1, keepdims=True)) @ vals


def attention_values_misaligned(q, keys, vals, scale):
    if keys.shape[0] == 0:
        return np.zeros((q.shape[0], vals.shape[1]))
    z = float(scale) * (q @ keys.T)
    w = np.exp(z - z.max(axis=1, keepdims=True))
    return (w / w.sum(axis=1, keepdims=True)) @ vals[::-1]


def attention_max_over_heads(q, keys, vals, scale):
    if keys.shape[0] == 0:
        return np.zeros((q.shape[0], vals.shape[1]))
    z = float(scale) * (q @ keys.T)
    w = np.exp(z - z.max(axis=0, keepdims=True))
    return (w / w.sum(axis=0, keepdims=True)) @ vals


def selected_tokens_whole_pages(pages, sel, n, page_size=PAGE):
    if len(sel) == 0:
        return np.zeros((0, pages.shape[2]))
    return np.concatenate([pages[int(p)] for p in sel], axis=0)


def merge_inverted_weights(parts):
    ms = np.stack([p[0] for p in parts])
    M = ms.max(axis=0)
    num, den = 0.0, 0.0
    for m, l, acc in parts:
        f = np.where(np.isfinite(m), np.exp(M - m), 0.0)
        num = num + f[:, None] * acc
        den = den + f * l
    return num / den[:, None]


def _votes(q_win, keys, n, scale, causal_shift=0, normalise=True, mask=True):
    G, W, D = q_win.shape
    L = n - W
    z = float(scale) * (q_win.reshape(G * W, D) @ keys[:n].T)
    pos = L + np.tile(np.arange(W), G)
    if mask:
        z = np.where(np.arange(n)[None, :] <= pos[:, None] + causal_shift, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    P = e / l if normalise else e
    return P[:, :L].sum(axis=0), m.reshape(G, W), l.reshape(G, W)


def votes_exclude_current_token(q_win, keys, n, scale):
    return _votes(q_win, keys, n, scale, causal_shift=-1)


def votes_without_causal_mask(q_win, keys, n, scale):
    return _votes(q_win, keys, n, scale, mask=False)


def votes_unnormalised(q_win, keys, n, scale):
    return _votes(q_win, keys, n, scale, normalise=False)


def pool_too_wide(S, kernel):
    r = kernel
    return np.array([S[max(0, j - r):j + r + 1].max() for j in range(len(S))])


def pool_one_sided(S, kernel):
    return np.array([S[j:j + kernel].max() for j in range(len(S))])


def keep_without_window(pooled, n, window, budget):
    L = n - window
    if L <= budget:
        return np.arange(n, dtype=np.int64)
    return oracle.unit_select(pooled, budget)


def keep_window_shifted(pooled, n, window, budget):
    L = n - window
    if L <= budget:
        return np.arange(n, dtype=np.int64)
    return np.concatenate([oracle.unit_select(pooled, budget), np.arange(L - 1, n - 1, dtype=np.int64)])


def decode_rows_one_short(q, keys_bits, vals_bits, length, group, scale):
    return oracle.dense_attention(oracle.bf16_to_f64(q), oracle.bf16_to_f64(np.asarray(keys_bits)[:, :length - 1]),
                                  oracle.bf16_to_f64(np.asarray(vals_bits)[:, :length - 1]), group, scale)


def candidates_recent_not_widened(n, window, sink=0, recent=0, interval=None):
    lo, hi = int(sink), int(n) - int(recent)
    if interval is not None:
        lo, hi = max(lo, int(interval[0])), min(hi, int(interval[1]))
    return lo, hi


def candidates_sink_one_past(n, window, sink=0, recent=0, interval=None):
    lo, hi = int(sink) + 1, int(n) - max(int(recent), int(window))
    if interval is not None:
        lo, hi = max(lo, int(interval[0])), min(hi, int(interval[1]))
    return lo, hi


def candidates_interval_end_inclusive(n, window, sink=0, recent=0, interval=None):
    lo, hi = int(sink), int(n) - max(int(recent), int(window))
    if interval is not None:
        lo, hi = max(lo, int(interval[0])), min(hi, int(interval[1]) + 1)
    return lo, hi


_true_keep = oracle.eviction_unit_keep


def keep_forced_inside_budget(pooled, n, window, budget, sink=0, recent=0, interval=None):
    lo, hi = oracle.eviction_candidates(n, window, sink, recent, interval)
    return _true_keep(pooled, n, window, max(budget - lo, 1), sink, recent, interval)


def keep_candidates_from_zero(pooled, n, window, budget, sink=0, recent=0, interval=None):
    lo, hi = oracle.eviction_candidates(n, window, sink, recent, interval)
    if hi - lo <= budget:
        return np.arange(n, dtype=np.int64)
    top = oracle.unit_select(np.asarray(pooled)[lo:hi], budget)  # offset forgotten
    return np.unique(np.concatenate([np.arange(lo), top, np.arange(hi, n)])).astype(np.int64)


_true_pyramid = oracle.pyramid_budgets


def pyramid_floors_only(num_layers, budget, ratio_first, ratio_last):
    L = int(num_layers)
    r = [ratio_first + (ratio_last - ratio_first) * l / max(L - 1, 1) for l in range(L)]
    return [int(L * budget * x / sum(r)) for x in r]


def pyramid_ratios_reversed(num_layers, budget, ratio_first, ratio_last):
    return _true_pyramid(num_layers, budget, ratio_last, ratio_first)


_true_compact = oracle.snapkv_compact


def compact_positions_ignored(*args, positions=None, **kw):
    return _true_compact(*args, **kw)


MUTANTS = {
    "bound: min instead of max": ("unit_page_bounds", bound_min_instead_of_max),
    "bound: dropped min term": ("unit_page_bounds", bound_max_term_only),
    "bound: missing scale": ("unit_page_bounds", bound_without_scale),
    "bound: split-sign halves swapped": ("unit_page_bounds", bound_split_sign_swapped),
    "head score: sum": ("unit_kv_head_score", head_score_sum),
    "head score: mean": ("unit_kv_head_score", head_score_mean),
    "select: ties to higher id": ("unit_select", select_ties_to_higher_id),
    "select: score order": ("unit_select", select_in_score_order),
    "select: one short": ("unit_select", select_one_short),
    "forced: pages counted inside the budget": ("unit_select_forced", forced_inside_budget),
    "forced: recent one page short": ("unit_select_forced", forced_recent_one_short),
    "summaries: whole last page": ("unit_summaries", summaries_over_whole_last_page),
    "summaries: last valid token dropped": ("unit_summaries", summaries_drop_last_valid_token),
    "attention: missing scale": ("unit_attention", attention_without_scale),
    "attention: values misaligned": ("unit_attention", attention_values_misaligned),
    "attention: softmax over heads": ("unit_attention", attention_max_over_heads),
    "gather: whole pages": ("unit_selected_tokens", selected_tokens_whole_pages),
    "merge: inverted weights": ("merge_partials", merge_inverted_weights),
    "votes: current token excluded": ("snapkv_unit_votes", votes_exclude_current_token),
    "votes: no causal mask": ("snapkv_unit_votes", votes_without_causal_mask),
    "votes: unnormalised rows": ("snapkv_unit_votes", votes_unnormalised),
    "pool: too wide": ("maxpool1d", pool_too_wide),
    "pool: one-sided": ("maxpool1d", pool_one_sided),
    "keep: window dropped": ("snapkv_unit_keep", keep_without_window),
    "keep: window shifted": ("snapkv_unit_keep", keep_window_shifted),
    "decode: one row short": ("decode_over_rows", decode_rows_one_short),
    "evict: recent not widened to the window": ("eviction_candidates", candidates_recent_not_widened),
    "evict: sink one past": ("eviction_candidates", candidates_sink_one_past),
    "evict: interval end inclusive": ("eviction_candidates", candidates_interval_end_inclusive),
    "evict: forced positions counted in the budget": ("eviction_unit_keep", keep_forced_inside_budget),
    "evict: candidate offset forgotten": ("eviction_unit_keep", keep_candidates_from_zero),
    "pyramid: floors only": ("pyramid_budgets", pyramid_floors_only),
    "pyramid: ratios reversed": ("pyramid_budgets", pyramid_ratios_reversed),
    "re-evict: positions ignored": ("snapkv_compact", compact_positions_ignored),
}


def test_unmutated_oracle_passes_every_pin():
    for pin in _pins():
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name):
    attr, wrong = MUTANTS[name]
    caught = []
    with mock.patch.object(oracle, attr, wrong):
        for pin in _pins():
            try:
                pin()
            except Exception as e:  # an assertion, or an error the mistake provokes
                caught.append(type(e).__name__)
                break
    assert caught, f"no pin fails with the planted mistake '{name}'"
