"""Pins for the eviction family around SnapKV's scores (O8) and PyramidKV's
per-layer budgets (O9).

Checks against the hand-worked example W3, the pairwise-order definition of a
selection (every kept candidate outranks every dropped one), the reduction to
plain SnapKV (O6, pinned by W2), exact rational shares for the budgets, and
bitwise row copies under re-eviction.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import test_oracle_snapkv as ts

HERE = os.path.dirname(__file__)
W3 = json.load(open(os.path.join(HERE, "golden", "eviction_w3.json")))


def test_worked_example_w3():
    n, W, pooled = W3["n"], W3["window"], np.array(W3["pooled"], dtype=np.float64)
    for c in W3["cases"]:
        iv = tuple(c["interval"]) if c["interval"] else None
        keep = oracle.eviction_unit_keep(pooled, n, W, c["budget"], c["sink"], c["recent"], iv)
        assert keep.tolist() == c["kept"], c["name"]
        cap = oracle.eviction_kept_capacity(n, W, c["budget"], c["sink"], c["recent"], iv)
        assert cap == c["kept_capacity"], c["name"]


def check_selection_definition(pooled, n, W, R, sink, recent, iv, keep):
    lo = sink
    hi = n - max(recent, W)
    if iv is not None:
        lo, hi = max(lo, iv[0]), min(hi, iv[1])
    kept = set(keep.tolist())
    assert (np.diff(keep) > 0).all() and len(kept) == len(keep)
    assert all(0 <= j < n for j in kept)
    outside = [j for j in range(n) if j < lo or j >= hi]
    assert set(outside) <= kept, "a position outside the candidate range was dropped"
    cand = [j for j in range(max(lo, 0), max(hi, lo))]
    if len(cand) <= R:
        assert len(kept) == n
        return
    chosen = [j for j in cand if j in kept]
    dropped = [j for j in cand if j not in kept]
    assert len(chosen) == R
    for i in chosen:
        for j in dropped:
            assert pooled[i] > pooled[j] or (pooled[i] == pooled[j] and i < j)


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000), n=st.integers(1, 60), W=st.integers(1, 6), R=st.integers(1, 20),
       sink=st.integers(0, 8), recent=st.integers(0, 12), use_iv=st.booleans(), ib=st.integers(0, 40),
       span=st.integers(1, 40), levels=st.sampled_from([2, 3, 50]))
def test_selection_against_pairwise_order(seed, n, W, R, sink, recent, use_iv, ib, span, levels):
    rng = np.random.default_rng(seed)
    L = max(n - W, 0)
    pooled = rng.integers(0, levels, L).astype(np.float64)  # few levels: ties on purpose
    iv = (ib, ib + span) if use_iv else None
    keep = oracle.eviction_unit_keep(pooled, n, W, R, sink, recent, iv)
    check_selection_definition(pooled, n, W, R, sink, recent, iv, keep)
    assert len(keep) <= oracle.eviction_kept_capacity(n + 5, W, R, sink, recent, iv)


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 10_000), n=st.integers(1, 60), W=st.integers(1, 6), R=st.integers(1, 20))
def test_defaults_reduce_to_snapkv(seed, n, W, R):
    rng = np.random.default_rng(seed)
    pooled = rng.integers(0, 4, max(n - W, 0)).astype(np.float64)
    a = oracle.eviction_unit_keep(pooled, n, W, R)
    b = oracle.snapkv_unit_keep(pooled, n, W, R)
    assert a.tolist() == b.tolist()
    # a recent budget no longer than the window, or an interval that covers the
    # whole prefix, changes nothing
    assert oracle.eviction_unit_keep(pooled, n, W, R, recent=W).tolist() == b.tolist()
    assert oracle.eviction_unit_keep(pooled, n, W, R, interval=(0, n + 3)).tolist() == b.tolist()
    assert oracle.eviction_kept_capacity(n, W, R) == R + W


def test_compact_with_forced_positions_and_interval():
    rng = np.random.default_rng(21)
    q, k, v, lens = ts.make_case(rng, lens=(80, 66))
    W, kern, G, s = 4, 5, 2, 0.35
    for sink, recent, R, iv in [(3, 9, 10, None), (0, 0, 6, (20, 50)), (5, 4, 7, (2, 70)), (0, 30, 12, None)]:
        cap = oracle.eviction_kept_capacity(80, W, R, sink, recent, iv)
        k_out, v_out, kept, kept_len, pooled = oracle.snapkv_compact(q, k, v, lens, G, s, W, kern, R, cap,
                                                                     sink=sink, recent=recent, interval=iv)
        assert kept.shape[2] == cap
        for b, n in enumerate(lens):
            for g in range(2):
                kl = int(kept_len[b, g])
                kk = kept[b, g, :kl]
                assert (kept[b, g, kl:] == -1).all()
                if pooled[b][g] is None:
                    assert kk.tolist() == list(range(n))
                else:
                    # the pooled vector is the pooled vote of brute-force votes
                    qw = oracle.bf16_to_f64(q[b, G * g:G * g + G])
                    Sb, _ = ts.brute_votes(qw, oracle.bf16_to_f64(k[b, g]), n, s)
                    np.testing.assert_allclose(pooled[b][g], oracle.maxpool1d(Sb, kern), rtol=1e-12)
                    check_selection_definition(pooled[b][g], n, W, R, sink, recent, iv, kk)
                np.testing.assert_array_equal(k_out[b, g, :kl], k[b, g, kk])
                np.testing.assert_array_equal(v_out[b, g, :kl], v[b, g, kk])


def test_reeviction_reports_original_positions():
    rng = np.random.default_rng(22)
    q, k, v, lens = ts.make_case(rng, lens=(80, 71))
    W, kern, G, s, R = 4, 3, 2, 0.35, 9
    cap = oracle.eviction_kept_capacity(80, W, R)
    plain = oracle.snapkv_compact(q, k, v, lens, G, s, W, kern, R, cap)
    ident = np.broadcast_to(np.arange(80), (2, 2, 80))
    same = oracle.snapkv_compact(q, k, v, lens, G, s, W, kern, R, cap, positions=ident)
    for a, b in zip(plain[:4], same[:4]):
        np.testing.assert_array_equal(a, b)
    # rows that stand for strictly increasing original positions
    pos = np.sort(rng.choice(10_000, size=(2, 2, 80), replace=False), axis=2)
    moved = oracle.snapkv_compact(q, k, v, lens, G, s, W, kern, R, cap, positions=pos)
    np.testing.assert_array_equal(moved[0], plain[0])
    np.testing.assert_array_equal(moved[1], plain[1])
    np.testing.assert_array_equal(moved[3], plain[3])
    for b in range(2):
        for g in range(2):
            kl = int(plain[3][b, g])
            rows = plain[2][b, g, :kl]
            assert moved[2][b, g, :kl].tolist() == pos[b, g, rows].tolist()
            assert (moved[2][b, g, kl:] == -1).all()
    # a budget that covers every candidate keeps the cache as it is, positions included
    whole = oracle.snapkv_compact(q, k, v, lens, G, s, W, kern, 80, 84, positions=pos)
    for b, n in enumerate(lens):
        assert whole[2][b, 0, :n].tolist() == pos[b, 0, :n].tolist()
        np.testing.assert_array_equal(whole[0][b, 0, :n], k[b, 0, :n])


def test_pyramid_worked_examples():
    for c in W3["pyramid"]:
        got = oracle.pyramid_budgets(c["layers"], c["budget"], c["ratio_first"], c["ratio_last"])
        assert got == c["budgets"], c["derivation"]


@settings(max_examples=60, deadline=None)
@given(L=st.integers(1, 96), R=st.integers(1, 20_000), a=st.floats(0.001, 1.0), z=st.floats(0.001, 1.0))
def test_pyramid_exact_shares(L, R, a, z):
    got = oracle.pyramid_budgets(L, R, a, z)
    assert len(got) == L and sum(got) == L * R
    A, Z = Fraction(round(a * 1e9), 10**9), Fraction(round(z * 1e9), 10**9)
    r = [A] if L == 1 else [A + (Z - A) * Fraction(l, L - 1) for l in range(L)]
    share = [Fraction(L * R) * x / sum(r) for x in r]
    for b, e in zip(got, share):
        assert e - 1 < b < e + 1
    assert all(b >= 0 for b in got)
    if a >= z:
        assert all(got[i] >= got[i + 1] - 1 for i in range(L - 1))


def test_pyramid_special_cases():
    assert oracle.pyramid_budgets(1, 4096, 0.6, 0.01) == [4096]
    assert oracle.pyramid_budgets(8, 100, 0.3, 0.3) == [100] * 8
    got = oracle.pyramid_budgets(47, 4096, 0.6, 0.01)  # Tables 8-9's ratios over a 47-layer stack
    assert sum(got) == 47 * 4096 and got[0] > got[-1] and got == sorted(got, reverse=True)
    assert got[0] / got[-1] == pytest.approx(60, rel=0.01)
