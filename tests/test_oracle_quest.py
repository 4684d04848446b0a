"""Pins for the Quest half of the oracle (O1-O5 and the split merge).

Nothing here re-types the oracle's formulas: each test checks the oracle
against a hand-worked example, brute force written differently, a library
routine (torch's float64 scaled-dot-product attention), a closed form or an
invariant that the pages' description implies.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from synth import bf16_bits

HERE = os.path.dirname(__file__)


def bits(x):
    return bf16_bits(torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def decode_torch(u16):
    """bf16 bits -> float64 through torch's own dtype (independent of the oracle's shift)."""
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(torch.float64)


def random_case(rng, B=2, Hkv=2, G=2, D=8, lens=(37, 16), ps=16, poison=True, pool_extra=3):
    MP = max(oracle.pages_of(n, ps) for n in lens) + 1
    pool = B * MP + pool_extra
    perm = rng.permutation(pool)
    table = perm[:B * MP].reshape(B, MP).astype(np.int32)
    k = bits(rng.standard_normal((pool, Hkv, ps, D)))
    v = bits(rng.standard_normal((pool, Hkv, ps, D)))
    if poison:
        for b, n in enumerate(lens):
            if n % ps:
                k[table[b, n // ps], :, n % ps:] = 0x7FC0
                v[table[b, n // ps], :, n % ps:] = 0x7FC0
    q = bits(rng.standard_normal((B, Hkv * G, D)))
    return q, k, v, table, np.array(lens, dtype=np.int32)


def dense_rows(pages, table_row, g, n, ps):
    """Token rows 0..n-1 of one head, read one token at a time through the page table."""
    rows = [pages[table_row[t // ps], g, t % ps] for t in range(n)]
    return np.stack(rows) if rows else np.zeros((0, pages.shape[-1]), np.uint16)


# ---------------------------------------------------------------------------
def test_bf16_decoding_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x4049], np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, -math.inf, 2.0 ** -133, 3.140625]
    got = oracle.bf16_to_f64(pats)
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)
    assert np.isnan(oracle.bf16_to_f64(np.array([0x7FC0], np.uint16)))[0]


def test_worked_example_w1():
    fx = json.load(open(os.path.join(HERE, "golden", "quest_w1.json")))
    ps, s = fx["page_size"], fx["scale"]
    keys = np.array(fx["keys"]).reshape(2, 1, ps, 2)
    vals = np.array(fx["values"]).reshape(2, 1, ps, 2)
    # store the two logical pages swapped in the pool to exercise the page table
    k = bits(keys[::-1].copy())
    v = bits(vals[::-1].copy())
    table = np.array([[1, 0]], np.int32)
    lens = np.array([4], np.int32)
    q = bits(np.array(fx["q"]).reshape(1, 1, 2))

    summ = oracle.quest_summaries(k, table, lens, ps)
    assert summ[0, 0, 0].tolist() == [[-1, 0], [1, 1]]
    assert summ[0, 1, 0].tolist() == [[0, -1], [2, 1]]
    A = oracle.quest_scores(q, summ, lens, 1, s, ps)
    assert A[0, 0].tolist() == [1.0, 4.0]

    e = math.e
    out1, sel1, _ = oracle.sparse_decode(q, k, v, table, lens, 1, 1, s, 2, page_size=ps)
    assert [list(x) for x in sel1[0]] == [[1]]
    np.testing.assert_allclose(out1[0, 0], [e**2 / (e**2 + 1), 1 / (e**2 + 1)], rtol=0, atol=1e-15)
    out2, sel2, _ = oracle.sparse_decode(q, k, v, table, lens, 2, 1, s, 2, page_size=ps)
    assert [list(x) for x in sel2[0]] == [[0, 1]]
    Z = e + e**-3 + e**2 + 1
    np.testing.assert_allclose(out2[0, 0], [e**2 / Z, 1 / Z], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out2[0, 0], [0.6622724, 0.0896288], atol=5e-8)


def test_summaries_brute_force():
    rng = np.random.default_rng(1)
    for ps, lens in ((16, (37, 16)), (16, (1, 47)), (4, (9, 12))):
        q, k, v, table, lens = random_case(rng, lens=lens, ps=ps)
        summ = oracle.quest_summaries(k, table, lens, ps)
        for b, n in enumerate(lens):
            P = -(-int(n) // ps)
            assert np.isnan(summ[b, P:]).all()
            for p in range(P):
                for g in range(k.shape[1]):
                    for c in range(k.shape[3]):
                        vals = [float(decode_torch(k[table[b, p], g, t - p * ps, c])) for t in range(p * ps, min(n, p * ps + ps))]
                        assert summ[b, p, g, 0, c] == min(vals)
                        assert summ[b, p, g, 1, c] == max(vals)


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 10_000), D=st.sampled_from([2, 4, 8, 64]), G=st.sampled_from([1, 2, 4, 8]),
       n=st.integers(1, 200), scale=st.floats(0.05, 3.0))
def test_bound_is_an_upper_bound_of_every_logit(seed, D, G, n, scale):
    rng = np.random.default_rng(seed)
    ps = 16
    q, k, v, table, lens = random_case(rng, B=1, Hkv=1, G=G, D=D, lens=(n,), ps=ps)
    summ = oracle.quest_summaries(k, table, lens, ps)
    qf = decode_torch(q).numpy()
    P = -(-n // ps)
    K = decode_torch(dense_rows(k, table[0], 0, n, ps)).numpy()
    for h in range(G):
        Uh = oracle.unit_page_bounds(qf[0, h:h + 1], summ[0, :P, 0, 0], summ[0, :P, 0, 1], scale)[0]
        for p in range(P):
            logits = scale * (K[p * ps:min(n, p * ps + ps)] @ qf[0, h])
            tol = 1e-12 * scale * np.abs(qf[0, h]).sum() * np.abs(K).max()
            assert Uh[p] >= logits.max() - tol
    A = oracle.quest_scores(q, summ, lens, G, scale, ps)
    for p in range(P):
        per_head = [oracle.unit_page_bounds(qf[0, h:h + 1], summ[0, p:p + 1, 0, 0], summ[0, p:p + 1, 0, 1], scale)[0, 0]
                    for h in range(G)]
        assert A[0, 0, p] == max(per_head)


def test_bound_tight_on_single_key_pages_and_zero_query():
    rng = np.random.default_rng(7)
    D, s = 16, 0.37
    q = bits(rng.standard_normal((1, 1, D)))
    k = bits(rng.standard_normal((3, 1, 16, D)))
    table = np.array([[2, 0, 1]], np.int32)
    lens = np.array([33], np.int32)  # last page holds one token
    # page 0: every slot the same key -> bound equals the logit exactly
    k[2, 0, :, :] = k[2, 0, 0, :]
    summ = oracle.quest_summaries(k, table, lens, 16)
    A = oracle.quest_scores(q, summ, lens, 1, s, 16)
    qf = decode_torch(q).numpy()[0, 0]
    for p, phys in ((0, 2), (2, 1)):
        key = decode_torch(k[phys, 0, 0]).numpy()
        assert A[0, 0, p] == pytest.approx(s * float(qf @ key), rel=1e-13, abs=1e-13)
    qz = np.zeros_like(q)
    Az = oracle.quest_scores(qz, summ, lens, 1, s, 16)
    assert (Az[0, 0, :3] == 0).all()


def test_kv_head_score_is_max_over_group():
    # two heads reading different channels of a page of identical keys (a, b)
    a, b, s = 3.0, -1.5, 0.5
    k = bits(np.tile(np.array([a, b]), (1, 1, 16, 1)))
    table = np.array([[0]], np.int32)
    lens = np.array([16], np.int32)
    q = bits(np.array([[[1.0, 0.0], [0.0, 1.0]]]))
    summ = oracle.quest_summaries(k, table, lens, 16)
    A = oracle.quest_scores(q, summ, lens, 2, s, 16)
    assert A[0, 0, 0] == s * max(a, b)
    Asum = oracle.quest_scores(q, summ, lens, 2, s, 16, mode="sum")
    assert Asum[0, 0, 0] == s * (a + b)


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000), P=st.integers(1, 60), topk=st.integers(1, 70), levels=st.integers(1, 6))
def test_selection_against_pairwise_order(seed, P, topk, levels):
    rng = np.random.default_rng(seed)
    scores = rng.integers(0, levels, P).astype(np.float64) - 2.5  # many exact ties
    sel = oracle.unit_select(scores, topk)
    k = min(topk, P)
    assert len(sel) == k and len(set(sel.tolist())) == k
    assert (np.diff(sel) > 0).all()
    inside = set(sel.tolist())
    for i in inside:
        for j in range(P):
            if j not in inside:
                # every kept id beats every dropped id: higher score, or equal score and lower id
                assert scores[i] > scores[j] or (scores[i] == scores[j] and i < j)


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000), P=st.integers(1, 40), topk=st.integers(0, 20), sink=st.integers(0, 6),
       recent=st.integers(0, 9), levels=st.integers(1, 5))
def test_forced_selection_against_its_definition(seed, P, topk, sink, recent, levels):
    """Sink and recent pages beside the selected budget (appendix Tables 8-11):
    the first `sink` and last `recent` pages are always kept, and among the
    other pages exactly min(topk, #others) are kept, each beating every dropped
    one (higher score, or equal score and lower id)."""
    rng = np.random.default_rng(seed)
    scores = rng.integers(0, levels, P).astype(np.float64) - 1.5  # many exact ties
    sel = oracle.unit_select_forced(scores, topk, sink, recent)
    assert (np.diff(sel) > 0).all()
    kept = set(sel.tolist())
    forced = {p for p in range(P) if p < sink or p >= P - recent}
    assert forced <= kept
    others = [p for p in range(P) if p not in forced]
    picked = kept - forced
    assert len(picked) == min(topk, len(others))
    for i in picked:
        for j in others:
            if j not in kept:
                assert scores[i] > scores[j] or (scores[i] == scores[j] and i < j)


def test_forced_selection_special_cases():
    rng = np.random.default_rng(31)
    for P in (1, 5, 17, 64):
        scores = rng.normal(size=P)
        # no forced pages: plain top-k
        for k in (1, 3, 70):
            assert oracle.unit_select_forced(scores, k, 0, 0).tolist() == oracle.unit_select(scores, k).tolist()
        # StreamingLLM: sink and recent only, no scoring budget
        assert oracle.unit_select_forced(scores, 0, 2, 3).tolist() == sorted(set(range(min(2, P))) |
                                                                                set(range(max(P - 3, 0), P)))
        # a budget covering the request keeps every page
        assert oracle.unit_select_forced(scores, P, 1, 1).tolist() == list(range(P))
    # worked case: 10 pages, sink 1, recent 2, budget 3 among pages 1..7
    scores = np.array([0.0, 5.0, 1.0, 7.0, 7.0, 2.0, 9.0, 3.0, -1.0, -2.0])
    assert oracle.unit_select_forced(scores, 3, 1, 2).tolist() == [0, 3, 4, 6, 8, 9]


@pytest.mark.parametrize("G,D,lens", [(1, 8, (37, 16)), (4, 64, (100, 1)), (8, 16, (200, 129))])
def test_dense_case_equals_library_attention(G, D, lens):
    rng = np.random.default_rng(G * 100 + D)
    ps = 16
    q, k, v, table, lens = random_case(rng, B=2, Hkv=2, G=G, D=D, lens=lens, ps=ps)
    MP = table.shape[1]
    out, sel, _ = oracle.sparse_decode(q, k, v, table, lens, MP, G, 0.3, D, page_size=ps)
    for b, n in enumerate(lens):
        for g in range(2):
            assert sel[b][g].tolist() == list(range(-(-int(n) // ps)))
            K = decode_torch(dense_rows(k, table[b], g, int(n), ps))[None, None]
            V = decode_torch(dense_rows(v, table[b], g, int(n), ps))[None, None]
            Q = decode_torch(q[b, g * G:(g + 1) * G])[None, :, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q, K.expand(1, G, -1, -1), V.expand(1, G, -1, -1), scale=0.3)[0, :, 0]
            np.testing.assert_allclose(out[b, g * G:(g + 1) * G], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_sparse_output_is_convex_combination_of_selected_rows():
    rng = np.random.default_rng(5)
    ps, G, D = 16, 4, 32
    q, k, v, table, lens = random_case(rng, B=1, Hkv=1, G=G, D=D, lens=(145,), ps=ps)
    out, sel, _ = oracle.sparse_decode(q, k, v, table, lens, 3, G, 0.2, D, page_size=ps)
    rows = []
    for p in sel[0][0]:
        for t in range(p * ps, min(145, p * ps + ps)):
            rows.append(decode_torch(v[table[0, p], 0, t - p * ps]).numpy())
    rows = np.stack(rows)
    assert (out[0] <= rows.max(0) + 1e-12).all() and (out[0] >= rows.min(0) - 1e-12).all()
    # a selection of the last page, which holds a single token, returns that value row exactly
    one = [[np.array([9])]]
    o1 = oracle.sparse_attention(q, k, v, table, lens, one, G, 0.2, D, page_size=ps)
    np.testing.assert_array_equal(o1[0], np.tile(decode_torch(v[table[0, 9], 0, 0]).numpy(), (G, 1)))


def test_split_merge_equals_single_softmax():
    rng = np.random.default_rng(11)
    qh = rng.standard_normal((3, 16))
    keys = rng.standard_normal((97, 16)) * 3
    vals = rng.standard_normal((97, 8))
    ref = oracle.unit_attention(qh, keys, vals, 0.7)
    for cuts in ([0, 97], [0, 40, 97], [0, 1, 2, 50, 96, 97], [0, 0, 30, 30, 97]):
        parts = [oracle.attention_partial(qh, keys[a:b], vals[a:b], 0.7) for a, b in zip(cuts[:-1], cuts[1:])]
        np.testing.assert_allclose(oracle.merge_partials(parts), ref, rtol=1e-12, atol=1e-12)


def test_heavy_token_pages_are_selected():
    from synth import TINY_QUEST, make_quest_inputs
    wl = TINY_QUEST.resized(context=1024, topk=12)
    x = make_quest_inputs(wl, "cpu")
    q, k = bf16_bits(x["q"]), bf16_bits(x["k_pages"])
    v = bf16_bits(x["v_pages"])
    table, lens = x["page_table"].numpy(), x["seq_lens"].numpy()
    _, sel, _ = oracle.sparse_decode(q, k, v, table, lens, wl.topk, wl.group, wl.scale, 64)
    # the heavy keys equal 4x the group's mean query: find them by brute force
    qbar = decode_torch(q[0]).numpy().mean(0)
    want = np.array(bf16_bits(torch.tensor(4 * qbar, dtype=torch.float32).to(torch.bfloat16)))
    heavy_pages = {p for p in range(64) for t in range(16) if (k[table[0, p], 0, t] == want).all()}
    assert len(heavy_pages) >= 1 and heavy_pages <= set(sel[0][0].tolist())
