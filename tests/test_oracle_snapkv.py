"""Pins for the SnapKV half of the oracle (O6, O7).

Checks against the hand-worked example W2, loop-by-loop brute force (plain
Python floats, no matmul), the closed form sum(votes) + window mass = G*W,
pooling and retention invariants, and bitwise compaction.
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


def dec(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def brute_votes(qw, keys, n, s):
    """Per-row softmax over j <= n-W+i with Python floats; returns (votes, window mass)."""
    G, W, D = qw.shape
    L = n - W
    votes = [0.0] * L
    window_mass = 0.0
    for h in range(G):
        for i in range(W):
            last = L + i
            logits = [s * math.fsum(qw[h, i, c] * keys[j, c] for c in range(D)) for j in range(last + 1)]
            mx = max(logits)
            ex = [math.exp(z - mx) for z in logits]
            tot = math.fsum(ex)
            for j in range(last + 1):
                if j < L:
                    votes[j] += ex[j] / tot
                else:
                    window_mass += ex[j] / tot
    return np.array(votes), window_mass


def test_worked_example_w2():
    fx = json.load(open(os.path.join(HERE, "golden", "snapkv_w2.json")))
    n, W, kern, R = fx["n"], fx["window"], fx["pool_kernel"], fx["budget"]
    keys = np.array(fx["keys"]).reshape(1, 1, n, 1)
    vals = np.array(fx["values"]).reshape(1, 1, n, 1)
    q = np.array(fx["q_window"]).reshape(1, 1, W, 1)
    e = math.e
    Z4, Z5 = 3 + e + e**2, 4 + e + e**2
    P4 = np.array([1, e**2, 1, e, 1]) / Z4
    P5 = np.array([1, e**2, 1, e, 1, 1]) / Z5
    S_want = P4[:4] + P5[:4]

    S, m, l = oracle.snapkv_unit_votes(oracle.bf16_to_f64(bits(q))[0], oracle.bf16_to_f64(bits(keys))[0, 0], n, 1.0)
    np.testing.assert_allclose(S, S_want, rtol=0, atol=1e-15)
    np.testing.assert_allclose(S, [0.147178, 1.087508, 0.147178, 0.400072], atol=1e-6)
    assert S.sum() + P4[4] + P5[4] + P5[5] == pytest.approx(2.0, abs=1e-15)
    pooled = oracle.maxpool1d(S, kern)
    np.testing.assert_array_equal(pooled, [S[1], S[1], S[1], S[3]])

    k_out, v_out, kept, kept_len, _ = oracle.snapkv_compact(bits(q), bits(keys), bits(vals), [n], 1, 1.0, W,
                                                             kern, R, 8)
    assert kept[0, 0].tolist() == [0, 1, 4, 5] and kept_len[0, 0] == 4
    assert dec(v_out[0, 0, :4, 0]).tolist() == [1.0, 2.0, 5.0, 6.0]
    assert (v_out[0, 0, 4:] == 0).all()


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 10_000), G=st.sampled_from([1, 2, 4]), W=st.integers(1, 5), L=st.integers(1, 30),
       D=st.sampled_from([1, 3, 8]), s=st.floats(0.1, 2.0))
def test_votes_brute_force_and_mass(seed, G, W, L, D, s):
    rng = np.random.default_rng(seed)
    n = L + W
    qw = oracle.bf16_to_f64(bits(rng.standard_normal((G, W, D))))
    keys = oracle.bf16_to_f64(bits(rng.standard_normal((n + 3, D)) * 2))
    S, m, l = oracle.snapkv_unit_votes(qw, keys, n, s)
    Sb, wmass = brute_votes(qw, keys, n, s)
    np.testing.assert_allclose(S, Sb, rtol=1e-12, atol=1e-14)
    assert S.sum() + wmass == pytest.approx(G * W, rel=1e-12)
    assert (S > 0).all()


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 10_000), L=st.integers(1, 40), kern=st.sampled_from([1, 3, 5, 7, 9]))
def test_maxpool_properties(seed, L, kern):
    rng = np.random.default_rng(seed)
    S = rng.integers(0, 5, L).astype(np.float64)
    P = oracle.maxpool1d(S, kern)
    assert (P >= S).all()
    if kern == 1:
        np.testing.assert_array_equal(P, S)
    # -inf padding formulation
    r = kern // 2
    padded = np.concatenate([np.full(r, -np.inf), S, np.full(r, -np.inf)])
    windows = np.lib.stride_tricks.sliding_window_view(padded, kern)
    np.testing.assert_array_equal(P, windows.max(axis=1))


def make_case(rng, B=2, Hkv=2, G=2, N=80, D=8, lens=(80, 61)):
    q = bits(rng.standard_normal((B, Hkv * G, 4, D)))
    k = bits(rng.standard_normal((B, Hkv, N, D)))
    v = bits(rng.standard_normal((B, Hkv, N, D)))
    return q, k, v, np.array(lens)


def test_identity_budget_keeps_everything_bitwise():
    rng = np.random.default_rng(3)
    q, k, v, lens = make_case(rng)
    W, R = 4, 80
    k_out, v_out, kept, kept_len, pooled = oracle.snapkv_compact(q, k, v, lens, 2, 0.35, W, 7, R, 96)
    for b, n in enumerate(lens):
        for g in range(2):
            assert kept_len[b, g] == n
            assert kept[b, g, :n].tolist() == list(range(n)) and (kept[b, g, n:] == -1).all()
            np.testing.assert_array_equal(k_out[b, g, :n], k[b, g, :n])
            np.testing.assert_array_equal(v_out[b, g, :n], v[b, g, :n])
            assert pooled[b][g] is None


def test_eviction_keeps_top_pooled_plus_window():
    rng = np.random.default_rng(4)
    q, k, v, lens = make_case(rng)
    W, R, kern = 4, 10, 7
    k_out, v_out, kept, kept_len, pooled = oracle.snapkv_compact(q, k, v, lens, 2, 0.35, W, kern, R, 16)
    for b, n in enumerate(lens):
        L = n - W
        for g in range(2):
            kk = kept[b, g, :kept_len[b, g]]
            assert kept_len[b, g] == R + W and (kept[b, g, R + W:] == -1).all()
            assert (np.diff(kk) > 0).all()
            assert kk[R:].tolist() == list(range(L, n))
            P = pooled[b][g]
            inside = set(kk[:R].tolist())
            for i in inside:
                for j in range(L):
                    if j not in inside:
                        assert P[i] > P[j] or (P[i] == P[j] and i < j)
            np.testing.assert_array_equal(k_out[b, g, :R + W], k[b, g, kk])
            np.testing.assert_array_equal(v_out[b, g, :R + W], v[b, g, kk])
            # the pooled vector is the pooled vote of brute-force votes
            qw = oracle.bf16_to_f64(q[b, 2 * g:2 * g + 2])
            Sb, _ = brute_votes(qw, oracle.bf16_to_f64(k[b, g]), n, 0.35)
            np.testing.assert_allclose(P, oracle.maxpool1d(Sb, kern), rtol=1e-12)


def test_decode_over_compacted_cache():
    rng = np.random.default_rng(9)
    q, k, v, lens = make_case(rng, lens=(80, 80))
    W, G = 4, 2
    # identity budget: decoding the compacted cache equals decoding the original
    k_id, v_id, _, klen, _ = oracle.snapkv_compact(q, k, v, lens, G, 0.35, W, 7, 200, 96)
    qd = bits(rng.standard_normal((4, 8)))
    a = oracle.decode_over_rows(qd, k_id[0], v_id[0], int(klen[0, 0]), G, 0.35)
    b = oracle.decode_over_rows(qd, k[0], v[0], 80, G, 0.35)
    np.testing.assert_array_equal(a, b)
    # with eviction: equals library attention over exactly the kept rows
    k_ev, v_ev, kept, klen, _ = oracle.snapkv_compact(q, k, v, lens, G, 0.35, W, 7, 12, 16)
    out = oracle.decode_over_rows(qd, k_ev[1], v_ev[1], 16, G, 0.35)
    for g in range(2):
        rows = kept[1, g, :16]
        K = torch.from_numpy(dec(k[1, g, rows]))[None, None]
        V = torch.from_numpy(dec(v[1, g, rows]))[None, None]
        Q = torch.from_numpy(dec(qd[g * G:(g + 1) * G]))[None, :, None]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K.expand(1, G, -1, -1), V.expand(1, G, -1, -1),
                                                               scale=0.35)[0, :, 0]
        np.testing.assert_allclose(out[g * G:(g + 1) * G], ref.numpy(), rtol=1e-12, atol=1e-12)
