"""GPU parity of the Quest path (summaries, scores, top-k, decode) against the
oracle, called through the C ABI, at sizes the oracle finishes in seconds.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_long_amd as se
from synth import QuestWorkload, TINY_QUEST, make_quest_inputs, bf16_bits
from gpu_util import (DEV, announce, build_summaries, check_attention, check_forced_selection, check_selection,
                      host_inputs, layout_for,
                      params_for, run_sparse_decode, score_tolerance, sel_lists, to_np, workspace)

pytestmark = pytest.mark.gpu

SMALL = {
    "d64_g4": (QuestWorkload("t_d64_g4", 2, 8, 2, 64, 64, 700, 12, "heavy", seed=11), [700, 333]),
    "d128_g8": (QuestWorkload("t_d128_g8", 3, 16, 2, 128, 128, 1500, 20, "zipf", seed=12), [1500, 1, 229]),
    "d128_g4_outlier": (QuestWorkload("t_d128_g4", 2, 16, 4, 128, 128, 2048, 16, "outlier", seed=13), [2048, 1000]),
    "d128_g1": (QuestWorkload("t_d128_g1", 2, 4, 4, 128, 128, 900, 10, "none", seed=14), [900, 17]),
    "d128_g2": (QuestWorkload("t_d128_g2", 1, 8, 4, 128, 128, 640, 7, "none", seed=15), [640]),
    "d128_g16": (QuestWorkload("t_d128_g16", 2, 32, 2, 128, 128, 800, 9, "none", seed=16), [800, 513]),
    "d128_g32": (QuestWorkload("t_d128_g32", 1, 32, 1, 128, 128, 1200, 11, "none", seed=17), [1199]),
    "d64_g16": (QuestWorkload("t_d64_g16", 1, 16, 1, 64, 64, 1000, 9, "none", seed=18), [1000]),
    "mla": (QuestWorkload("t_mla", 2, 32, 1, 576, 512, 1000, 16, "none", v_is_k_prefix=True, seed=19), [1000, 455]),
    "mla_g8": (QuestWorkload("t_mla_g8", 1, 8, 1, 576, 512, 600, 5, "none", v_is_k_prefix=True, seed=20), [600]),
    # a 40-page budget: with an even split count the latent-layout decode's
    # splits come in two halves of unequal length; the short requests leave
    # whole splits of either half empty
    "mla_k40": (QuestWorkload("t_mla_k40", 3, 32, 1, 576, 512, 2000, 40, "none", v_is_k_prefix=True, seed=24),
                [2000, 600, 17]),
}


def make(name, poison=True):
    wl, lens = SMALL[name]
    announce(f"quest case {name} seed {wl.seed} lens {lens}")
    return wl, make_quest_inputs(wl, DEV, poison_tail=poison, seq_lens=lens, pool_extra=5)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_summaries_exact(name):
    wl, x = make(name)
    summ = build_summaries(x, wl)
    torch.cuda.synchronize()
    h = host_inputs(x)
    ref = oracle.quest_summaries(h["k"], h["pt"], h["lens"])
    got = oracle.bf16_to_f64(bf16_bits(summ))
    for b, n in enumerate(h["lens"]):
        P = -(-int(n) // 16)
        phys = h["pt"][b, :P]
        np.testing.assert_array_equal(got[phys], ref[b, :P])
        # bitwise as well (the data holds no zeros whose sign could differ)
        ref_bits = (ref[b, :P].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        assert (bf16_bits(summ)[phys] == ref_bits).all()


@pytest.mark.parametrize("name", ["d64_g4", "d128_g8", "d128_g1", "d128_g16", "mla"])
@pytest.mark.parametrize("head_agg", [0, 1])
def test_scores_and_last_page_refresh(name, head_agg):
    wl, x = make(name)
    summ = build_summaries(x, wl)
    h = host_inputs(x)
    # corrupt every request's last-page summary; the refresh must rebuild it
    for b, n in enumerate(h["lens"]):
        P = -(-int(n) // 16)
        summ[int(h["pt"][b, P - 1])] = 3.0
    P = params_for(wl, refresh=1, head_agg=head_agg)
    scores = torch.full((wl.batch, wl.num_kv_heads, wl.max_pages), float("nan"), device=DEV)
    se.se_quest_scores(layout_for(wl), P, x["q"], x["k_pages"], x["page_table"], summ, x["seq_lens"], scores)
    torch.cuda.synchronize()
    ref_summ = oracle.quest_summaries(h["k"], h["pt"], h["lens"])
    got_summ = oracle.bf16_to_f64(bf16_bits(summ))
    A = oracle.quest_scores(h["q"], ref_summ, h["lens"], wl.group, wl.scale, mode="max" if head_agg == 0 else "sum")
    qf = oracle.bf16_to_f64(h["q"])
    S = to_np(scores)
    for b, n in enumerate(h["lens"]):
        Pb = -(-int(n) // 16)
        np.testing.assert_array_equal(got_summ[h["pt"][b, :Pb]], ref_summ[b, :Pb])
        for g in range(wl.num_kv_heads):
            if wl.topk >= Pb:
                assert np.isnan(S[b, g]).all(), "dense request must not be scored"
                continue
            tol = score_tolerance(qf[b, g * wl.group:(g + 1) * wl.group], ref_summ[b, :Pb, g, 0], ref_summ[b, :Pb, g, 1],
                                  wl.scale)
            if head_agg == 1:
                tol = tol * wl.group
            err = np.abs(S[b, g, :Pb] - A[b, g, :Pb])
            assert (err <= tol).all(), f"b{b} g{g}: worst {np.max(err / tol):.3f} of tolerance"
            assert np.isnan(S[b, g, Pb:]).all()


@pytest.mark.parametrize("MP,topk", [(5, 2), (300, 17), (1024, 64), (3000, 256), (9000, 300), (20000, 2048),
                                     (40000, 1000), (65536, 4096)])
def test_topk_pages_exact(MP, topk):
    announce(f"topk MP {MP} topk {topk}")
    rng = np.random.default_rng(MP + topk)
    B, Hkv = 3, 2
    scores = rng.standard_normal((B, Hkv, MP)).astype(np.float32)
    scores[0, 0] = rng.integers(0, 7, MP)  # heavy ties
    scores[1, 1, ::3] = -0.0
    scores[1, 1, 1::3] = 0.0
    scores[2, 0] = 1.5  # every key equal
    scores[2, 1] = np.float32(3.0) * (1 + (np.arange(MP) % 5 == 0))  # keys sharing their top bits
    lens = np.array([MP * 16, MP * 16 - 5, max(1, MP * 8)], np.int32)
    P = se.decode_params(B, Hkv, MP, topk)
    sel = torch.full((B, Hkv, topk), 12345, dtype=torch.int32, device=DEV)
    se.se_topk_pages(P, Hkv, torch.from_numpy(scores).to(DEV), torch.from_numpy(lens).to(DEV), sel)
    torch.cuda.synchronize()
    got = to_np(sel)
    for b in range(B):
        Pb = -(-int(lens[b]) // 16)
        for g in range(Hkv):
            want = oracle.unit_select(scores[b, g, :Pb].astype(np.float64), topk)
            k = len(want)
            assert (got[b, g, :k] == want).all(), f"b{b} g{g}"
            assert (got[b, g, k:] == -1).all()


def _decode_case(name, topk=None, splits=0, valu=0):
    wl, x = make(name)
    summ = build_summaries(x, wl)
    out, sel = run_sparse_decode(x, wl, summ, topk=topk, refresh=1, splits=splits, valu=valu)
    h = host_inputs(x)
    ref_summ = oracle.quest_summaries(h["k"], h["pt"], h["lens"])
    A = oracle.quest_scores(h["q"], ref_summ, h["lens"], wl.group, wl.scale)
    sel_np = to_np(sel)
    k = wl.topk if topk is None else topk
    for b, n in enumerate(h["lens"]):
        Pb = -(-int(n) // 16)
        for g in range(wl.num_kv_heads):
            check_selection(sel_np[b, g], A[b, g, :Pb], k, f"{name} b{b} g{g}")
    ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], sel_lists(sel_np, h["lens"]), wl.group,
                                  wl.scale, wl.head_dim_v, wl.v_is_k_prefix)
    return wl, x, out, sel, ref


@pytest.mark.parametrize("name", sorted(SMALL))
def test_sparse_decode_matches_oracle(name):
    wl, x, out, sel, ref = _decode_case(name)
    vmax = float(torch.nan_to_num(x["v_pages"] if x["v_pages"] is not None else x["k_pages"], 0.0).abs().max())
    check_attention(to_np(out), ref, vmax, name)


@pytest.mark.parametrize("splits", [2, 3, 4, 8, 16])
def test_latent_decode_split_halves_match_oracle(splits):
    """Even split counts put the latent-layout decode's splits in two halves,
    the first with longer splits (40 pages over 4 splits: 11 + 11 + 9 + 9;
    over 16: eight of 3 and eight of 2); odd counts keep equal splits.  Selection by the gap rule and attention against the
    oracle, for requests of 125, 38 and 2 pages."""
    wl, x, out, sel, ref = _decode_case("mla_k40", splits=splits)
    vmax = float(torch.nan_to_num(x["k_pages"], 0.0).abs().max())
    check_attention(to_np(out), ref, vmax, f"mla_k40 splits {splits}")


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("name", ["d128_g8", "d128_g16", "d128_g4_outlier", "d128_g1", "mla", "mla_g8", "d64_g4"])
def test_valu_attention_matches_oracle(name, splits):
    """valu_attention = 1: the vector-ALU attention kernel also on the shapes
    that otherwise run on the matrix cores (head dim 128 with up to 16 query
    heads per KV head, the 576/512 latent layout), with the automatic, one
    and three splits."""
    wl, x, out, sel, ref = _decode_case(name, splits=splits, valu=1)
    vmax = float(torch.nan_to_num(x["v_pages"] if x["v_pages"] is not None else x["k_pages"], 0.0).abs().max())
    check_attention(to_np(out), ref, vmax, f"{name} valu splits {splits}")


def test_budget_beyond_a_thousand_splits():
    """Head dim 64 with 32 query heads per KV head stages at most 16 pages per
    split; 18,000 kept pages of 20,000 need 1,125 splits, more than the split
    count could reach before (such a call used to pass the host checks and
    fail at launch)."""
    wl = QuestWorkload("t_many_splits", 1, 32, 1, 64, 64, 20000 * 16, 18000, "none", seed=24)
    announce(f"many splits seed {wl.seed}")
    x = make_quest_inputs(wl, DEV, poison_tail=True, seq_lens=[20000 * 16 - 3])
    summ = build_summaries(x, wl)
    out, sel = run_sparse_decode(x, wl, summ)
    h = host_inputs(x)
    ref_summ = oracle.quest_summaries(h["k"], h["pt"], h["lens"])
    A = oracle.quest_scores(h["q"], ref_summ, h["lens"], wl.group, wl.scale)
    sel_np = to_np(sel)
    check_selection(sel_np[0, 0], A[0, 0, :20000], wl.topk, "many splits")
    ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], sel_lists(sel_np, h["lens"]), wl.group,
                                  wl.scale, wl.head_dim_v)
    check_attention(to_np(out), ref, float(x["v_pages"].float().abs().max()), "many splits")


def test_tiny_quest_workload_full_size():
    """The tiny 4K-token workload runs at its full size; heavy pages are kept."""
    wl = TINY_QUEST
    announce(f"tiny quest full size seed {wl.seed}")
    x = make_quest_inputs(wl, DEV)
    summ = build_summaries(x, wl)
    out, sel = run_sparse_decode(x, wl, summ)
    h = host_inputs(x)
    ref_out, ref_sel, A = oracle.sparse_decode(h["q"], h["k"], h["v"], h["pt"], h["lens"], wl.topk, wl.group, wl.scale,
                                               wl.head_dim_v)
    sel_np = to_np(sel)
    check_selection(sel_np[0, 0], A[0, 0], wl.topk, "tiny")
    ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], sel_lists(sel_np, h["lens"]), wl.group,
                                  wl.scale, wl.head_dim_v)
    check_attention(to_np(out), ref, float(x["v_pages"].float().abs().max()), "tiny")


@pytest.mark.parametrize("name", ["d64_g4", "d128_g8", "mla"])
def test_dense_mode_equals_full_attention(name):
    wl, x = make(name)
    MP = wl.max_pages
    out, sel = run_sparse_decode(x, wl, None, topk=MP, refresh=0)
    h = host_inputs(x)
    full = [[np.arange(-(-int(n) // 16)) for _ in range(wl.num_kv_heads)] for n in h["lens"]]
    ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], full, wl.group, wl.scale, wl.head_dim_v,
                                  wl.v_is_k_prefix)
    sel_np = to_np(sel)
    for b, n in enumerate(h["lens"]):
        Pb = -(-int(n) // 16)
        assert (sel_np[b, :, :Pb] == np.arange(Pb)).all() and (sel_np[b, :, Pb:] == -1).all()
    check_attention(to_np(out), ref, 8.0, name)


@pytest.mark.parametrize("valu", [0, 1])
@pytest.mark.parametrize("name", ["d128_g8", "mla", "d64_g4"])
def test_split_count_invariance_and_determinism(name, valu):
    wl, x = make(name)
    summ = build_summaries(x, wl)
    base = summ.clone()
    outs = []
    # up to 16 splits the merge takes its one-round-trip path, above it the
    # LDS path (d128_g8 keeps 20 pages: 20 requested splits give 20)
    for splits in (1, 3, 16, 20, 0, 0):
        summ.copy_(base)
        o, s = run_sparse_decode(x, wl, summ, splits=splits, valu=valu)
        outs.append((to_np(o), to_np(s)))
    # the matrix-core decode carries each attention weight as a hi + lo pair of
    # bf16 (|error| <= 2^-16 of the weight), so two summation orders may differ
    # by up to 2 * 2^-16 * max|v|; allow 2^-14 * max|v|
    vmax = float(torch.nan_to_num(x["v_pages"] if x["v_pages"] is not None else x["k_pages"], 0.0).abs().max())
    for o, s in outs[1:]:
        assert (s == outs[0][1]).all()
        np.testing.assert_allclose(o, outs[0][0], rtol=0, atol=2.0**-14 * vmax)
    assert (outs[-2][0] == outs[-1][0]).all(), "repeated call not bitwise identical"


@pytest.mark.parametrize("name", ["d128_g8", "mla"])
def test_large_logit_range_matches_oracle(name):
    """Queries scaled by 16 spread the logits over a range of hundreds, so the
    decode's running max jumps by more than its lazy-rescale threshold on some
    pages and by less on others; the result still matches the oracle."""
    wl, x = make(name)
    x["q"] = (x["q"].float() * 16).to(torch.bfloat16)
    summ = build_summaries(x, wl)
    out, sel = run_sparse_decode(x, wl, summ, refresh=1)
    h = host_inputs(x)
    sel_np = to_np(sel)
    ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], sel_lists(sel_np, h["lens"]), wl.group,
                                  wl.scale, wl.head_dim_v, wl.v_is_k_prefix)
    vmax = float(torch.nan_to_num(x["v_pages"] if x["v_pages"] is not None else x["k_pages"], 0.0).abs().max())
    assert np.isfinite(to_np(out)).all()
    check_attention(to_np(out), ref, vmax, f"{name} q*16")


def test_mla_batch_beyond_one_scorer_launch():
    """2100 MLA units: more than one launch of the wide scorer's unit limit, each
    with its own last-page refreshes; selection and attention of every unit
    against the oracle."""
    wl = QuestWorkload("t_mla_many", 2100, 8, 1, 576, 512, 80, 2, "none", v_is_k_prefix=True, ragged_lo=17, seed=23)
    announce(f"mla many units seed {wl.seed}")
    x = make_quest_inputs(wl, DEV, poison_tail=True)
    summ = build_summaries(x, wl)
    out, sel = run_sparse_decode(x, wl, summ, refresh=1)
    h = host_inputs(x)
    ref_summ = oracle.quest_summaries(h["k"], h["pt"], h["lens"])
    A = oracle.quest_scores(h["q"], ref_summ, h["lens"], wl.group, wl.scale)
    sel_np = to_np(sel)
    for b, n in enumerate(h["lens"]):
        check_selection(sel_np[b, 0], A[b, 0, :-(-int(n) // 16)], wl.topk, f"mla many b{b}")
    ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], sel_lists(sel_np, h["lens"]), wl.group,
                                  wl.scale, wl.head_dim_v, wl.v_is_k_prefix)
    check_attention(to_np(out), ref, float(torch.nan_to_num(x["k_pages"], 0.0).abs().max()), "mla many")


@pytest.mark.parametrize("name", ["d128_g8", "mla", "d64_g4"])
def test_forced_sink_and_recent_pages_match_oracle(name):
    """Sink and recent pages kept beside the scored budget (appendix Tables
    8-11): forced pages exact, the others by the gap rule, attention against
    the oracle on the GPU's selection."""
    wl, x = make(name)
    summ = build_summaries(x, wl)
    sink, recent, topk = 1, 2, max(wl.topk // 2, 1)
    out, sel = run_sparse_decode(x, wl, summ, topk=topk, refresh=1, sink=sink, recent=recent)
    h = host_inputs(x)
    ref_summ = oracle.quest_summaries(h["k"], h["pt"], h["lens"])
    A = oracle.quest_scores(h["q"], ref_summ, h["lens"], wl.group, wl.scale)
    sel_np = to_np(sel)
    for b, n in enumerate(h["lens"]):
        Pb = -(-int(n) // 16)
        for g in range(wl.num_kv_heads):
            check_forced_selection(sel_np[b, g], A[b, g, :Pb], topk, sink, recent, f"{name} b{b} g{g}")
    ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], sel_lists(sel_np, h["lens"]), wl.group,
                                  wl.scale, wl.head_dim_v, wl.v_is_k_prefix)
    vmax = float(torch.nan_to_num(x["v_pages"] if x["v_pages"] is not None else x["k_pages"], 0.0).abs().max())
    check_attention(to_np(out), ref, vmax, f"{name} sink/recent")


@pytest.mark.parametrize("name", ["d128_g8", "mla"])
def test_sink_and_recent_only_needs_no_summaries(name):
    """topk = 0 keeps exactly the sink and recent pages (the StreamingLLM rows of
    appendix Tables 8-9), scores nothing and reads no summaries."""
    wl, x = make(name)
    sink, recent = 1, 3
    out, sel = run_sparse_decode(x, wl, None, topk=0, refresh=0, sink=sink, recent=recent)
    h = host_inputs(x)
    sel_np = to_np(sel)
    want = oracle.quest_select(np.zeros((wl.batch, wl.num_kv_heads, wl.max_pages)), h["lens"], 0, sink=sink,
                               recent=recent)
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            k = len(want[b][g])
            assert (sel_np[b, g, :k] == want[b][g]).all() and (sel_np[b, g, k:] == -1).all(), f"b{b} g{g}"
    ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], want, wl.group, wl.scale,
                                  wl.head_dim_v, wl.v_is_k_prefix)
    vmax = float(torch.nan_to_num(x["v_pages"] if x["v_pages"] is not None else x["k_pages"], 0.0).abs().max())
    check_attention(to_np(out), ref, vmax, f"{name} sink/recent only")


@pytest.mark.parametrize("splits", [0, 1, 2])
def test_empty_and_single_token_requests(splits):
    """Lengths 0, 1, 16 and 17 with the automatic split count, one split (the
    decode writes the output itself, no merge) and two."""
    wl = QuestWorkload("t_edge", 4, 8, 2, 128, 128, 64, 2, "none", seed=21)
    announce(f"edge lengths [0, 1, 16, 17], splits {splits}")
    x = make_quest_inputs(wl, DEV, poison_tail=True, seq_lens=[0, 1, 16, 17])
    summ = build_summaries(x, wl)
    out, sel = run_sparse_decode(x, wl, summ, splits=splits)
    o = to_np(out)
    assert (o[0] == 0).all()
    h = host_inputs(x)
    v0 = oracle.bf16_to_f64(h["v"][h["pt"][1, 0], :, 0, :])  # [Hkv, D]
    np.testing.assert_allclose(o[1], np.repeat(v0, wl.group, axis=0), rtol=0, atol=1e-6)
    ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], sel_lists(to_np(sel), h["lens"]),
                                  wl.group, wl.scale, wl.head_dim_v)
    check_attention(o, ref, 8.0, "edge")


def test_longest_supported_request():
    """One request at the largest page table the library takes (65536 pages,
    about 1M tokens, the last page partial), through the whole decode step."""
    wl = QuestWorkload("t_1m", 1, 8, 1, 128, 128, 65536 * 16, 512, "zipf", seed=23)
    n = 65536 * 16 - 5
    announce(f"longest request n {n}")
    x = make_quest_inputs(wl, DEV, poison_tail=True, seq_lens=[n])
    summ = build_summaries(x, wl)
    out, sel = run_sparse_decode(x, wl, summ)
    pt = to_np(x["page_table"])
    Pb = -(-n // 16)
    kbits = bf16_bits(x["k_pages"].index_select(0, torch.from_numpy(pt[0, :Pb].astype(np.int64)).to(DEV))[:, 0])
    kp = oracle.gather_unit_pages(kbits[:, None], np.arange(Pb), 0, n)
    mins, maxs = oracle.unit_summaries(kp, n)
    qf = oracle.bf16_to_f64(bf16_bits(x["q"])[0])
    A = oracle.unit_kv_head_score(oracle.unit_page_bounds(qf, mins, maxs, wl.scale))
    S = to_np(sel)
    check_selection(S[0, 0], A, wl.topk, "1M")
    chosen = S[0, 0].astype(np.int64)
    vbits = bf16_bits(x["v_pages"].index_select(0, torch.from_numpy(pt[0, chosen].astype(np.int64)).to(DEV))[:, 0])
    keys = oracle.unit_selected_tokens(kp, chosen, n)
    vp = np.full((Pb, 16, 128), np.nan)
    vp[chosen] = oracle.gather_unit_pages(vbits[:, None], np.arange(len(chosen)), 0, len(chosen) * 16)
    if chosen[-1] == Pb - 1:  # the partial last page keeps only its valid rows
        vp[Pb - 1, n - (Pb - 1) * 16:] = np.nan
    vals = oracle.unit_selected_tokens(vp, chosen, n)
    ref = oracle.unit_attention(qf, keys, vals, wl.scale)
    check_attention(to_np(out)[0], ref, float(np.abs(vals).max()), "1M")


@pytest.mark.parametrize("name", ["d128_g8", "mla"])
def test_shared_prefix_pages_match_oracle(name):
    """Requests whose page tables point at the same physical pages for a
    common prefix (a shared prompt): summaries stay per physical page and
    bitwise, every request's selection and attention follow the oracle on the
    same page table, and the refresh of each request's own last page leaves
    the shared pages as built."""
    base, _ = SMALL[name]
    wl = QuestWorkload(base.name + "_shared", 3, base.num_q_heads, base.num_kv_heads, base.head_dim_qk,
                       base.head_dim_v, base.context, base.topk, base.saliency, v_is_k_prefix=base.v_is_k_prefix,
                       seed=base.seed + 100)
    lens = [wl.context, wl.context - 37, wl.context - 300]
    shared = 30  # full pages in every request
    announce(f"quest shared prefix {name} seed {wl.seed} lens {lens} shared pages {shared}")
    x = make_quest_inputs(wl, DEV, poison_tail=True, seq_lens=lens, pool_extra=5)
    assert min(lens) > 16 * shared
    x["page_table"][1:, :shared] = x["page_table"][0, :shared]
    summ = build_summaries(x, wl)
    out, sel = run_sparse_decode(x, wl, summ)
    h = host_inputs(x)
    ref_summ = oracle.quest_summaries(h["k"], h["pt"], h["lens"])
    got = oracle.bf16_to_f64(bf16_bits(summ))
    for b, n in enumerate(h["lens"]):
        P = -(-int(n) // 16)
        np.testing.assert_array_equal(got[h["pt"][b, :P]], ref_summ[b, :P])
    A = oracle.quest_scores(h["q"], ref_summ, h["lens"], wl.group, wl.scale)
    sel_np = to_np(sel)
    for b, n in enumerate(h["lens"]):
        Pb = -(-int(n) // 16)
        for g in range(wl.num_kv_heads):
            check_selection(sel_np[b, g], A[b, g, :Pb], wl.topk, f"shared {name} b{b} g{g}")
    ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], sel_lists(sel_np, h["lens"]), wl.group,
                                  wl.scale, wl.head_dim_v, wl.v_is_k_prefix)
    vmax = float(torch.nan_to_num(x["v_pages"] if x["v_pages"] is not None else x["k_pages"], 0.0).abs().max())
    check_attention(to_np(out), ref, vmax, f"shared {name}")
