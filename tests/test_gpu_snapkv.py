"""GPU parity of the SnapKV path (votes, pool, select, compaction, decode over
the compacted cache) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_long_amd as se
from synth import SnapKVWorkload, make_snapkv_inputs, bf16_bits
from gpu_util import call_twice, DEV, announce, check_attention, check_selection, to_np, workspace

pytestmark = pytest.mark.gpu

SMALL = {
    "d128_g4_w32": (SnapKVWorkload("s_d128", 3, 8, 2, 128, 1000, 32, 7, 100, 4, seed=31), [1000, 700, 120]),
    "d64_g2_w8": (SnapKVWorkload("s_d64", 2, 4, 2, 64, 300, 8, 3, 40, 3, seed=32), [300, 47]),
    "d128_g32_w8": (SnapKVWorkload("s_g32", 1, 32, 1, 128, 500, 8, 7, 64, 2, seed=33), [500]),
    "d128_g1_w1": (SnapKVWorkload("s_w1", 2, 2, 2, 128, 400, 1, 5, 50, 2, seed=34), [400, 333]),
    "d128_g8_w24": (SnapKVWorkload("s_g8", 1, 8, 1, 128, 800, 24, 9, 200, 2, seed=35), [800]),
    # 16 heads x 128 window rows = 2048 rows: sixteen row groups, more than a
    # block's waves can take, so each row group gets blocks of its own
    "d64_g16_w128": (SnapKVWorkload("s_rows", 2, 16, 1, 64, 400, 128, 5, 60, 2, seed=37), [400, 250]),
    # empty prompt, shorter than the window, exactly the window, prefix == budget (identity),
    # prefix one past the budget, and a long one
    "edges": (SnapKVWorkload("s_edge", 6, 8, 2, 128, 300, 16, 5, 40, 2, seed=36), [0, 7, 16, 56, 57, 300]),
}


def make(name):
    wl, lens = SMALL[name]
    announce(f"snapkv case {name} seed {wl.seed} lens {lens}")
    return wl, make_snapkv_inputs(wl, DEV, prompt_lens=lens)


def params(wl):
    return se.snapkv_params(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.prompt, wl.window,
                            wl.pool_kernel, wl.budget, wl.out_capacity, wl.scale)


def host(x):
    return {"q": bf16_bits(x["q_win"]), "k": bf16_bits(x["k"]), "v": bf16_bits(x["v"]), "lens": to_np(x["prompt_lens"])}


def oracle_votes(h, wl, b, g):
    n = int(h["lens"][b])
    G = wl.group
    qw = oracle.bf16_to_f64(h["q"][b, g * G:(g + 1) * G])
    S, _, _ = oracle.snapkv_unit_votes(qw, oracle.bf16_to_f64(h["k"][b, g]), n, wl.scale)
    return S


@pytest.mark.parametrize("name", sorted(SMALL))
def test_votes_match_oracle(name):
    wl, x = make(name)
    p = params(wl)
    ws = workspace(se.se_snapkv_workspace_size(p))
    votes = torch.full((wl.batch, wl.num_kv_heads, wl.prompt), float("nan"), device=DEV)
    call_twice(lambda: se.se_snapkv_votes(p, x["q_win"], x["k"], x["prompt_lens"], votes, ws), ws, [votes],
               f"votes {name}")
    V = to_np(votes)
    h = host(x)
    for b, n in enumerate(h["lens"]):
        L = int(n) - wl.window
        for g in range(wl.num_kv_heads):
            if L <= 0:
                assert np.isnan(V[b, g]).all()
                continue
            S = oracle_votes(h, wl, b, g)
            err = np.abs(V[b, g, :L] - S)
            tol = 2e-4 * S + 1e-6 * S.max()
            assert (err <= tol).all(), f"b{b} g{g}: worst {np.max(err / tol):.3f} of tolerance"
            assert np.isnan(V[b, g, L:]).all()


@pytest.mark.parametrize("name", ["d128_g4_w32", "d64_g2_w8", "d128_g8_w24"])
def test_pool_and_select_exact_on_given_votes(name):
    wl, x = make(name)
    p = params(wl)
    rng = np.random.default_rng(wl.seed)
    votes = rng.integers(0, 9, (wl.batch, wl.num_kv_heads, wl.prompt)).astype(np.float32) / 8  # ties on purpose
    pooled = torch.full_like(torch.from_numpy(votes), float("nan")).to(DEV)
    se.se_maxpool1d(p, torch.from_numpy(votes).to(DEV), x["prompt_lens"], pooled)
    kept = torch.full((wl.batch, wl.num_kv_heads, wl.budget + wl.window), 777, dtype=torch.int32, device=DEV)
    klen = torch.zeros((wl.batch, wl.num_kv_heads), dtype=torch.int32, device=DEV)
    se.se_snapkv_select(p, pooled, x["prompt_lens"], kept, klen)
    torch.cuda.synchronize()
    Pg, K, KL = to_np(pooled), to_np(kept), to_np(klen)
    lens = to_np(x["prompt_lens"])
    for b, n in enumerate(lens):
        L = int(n) - wl.window
        for g in range(wl.num_kv_heads):
            if L > 0:
                want = oracle.maxpool1d(votes[b, g, :L].astype(np.float64), wl.pool_kernel)
                assert (Pg[b, g, :L] == want).all()
            keep = oracle.snapkv_unit_keep(Pg[b, g, :max(L, 0)].astype(np.float64), int(n), wl.window, wl.budget)
            assert KL[b, g] == len(keep)
            assert (K[b, g, :len(keep)] == keep).all() and (K[b, g, len(keep):] == -1).all()


def run_compact(wl, x):
    p = params(wl)
    ws = workspace(se.se_snapkv_workspace_size(p))
    B, H, C, D = wl.batch, wl.num_kv_heads, wl.out_capacity, wl.head_dim
    k_out = torch.zeros((B, H, C, D), dtype=torch.bfloat16, device=DEV)
    v_out = torch.zeros((B, H, C, D), dtype=torch.bfloat16, device=DEV)
    kept = torch.full((B, H, wl.budget + wl.window), 777, dtype=torch.int32, device=DEV)
    klen = torch.zeros((B, H), dtype=torch.int32, device=DEV)
    call_twice(lambda: se.se_snapkv_compact(p, x["q_win"], x["k"], x["v"], x["prompt_lens"], k_out, v_out, kept, klen,
                                            ws), ws, [k_out, v_out, kept, klen], f"compact {wl.name}")
    return k_out, v_out, kept, klen


@pytest.mark.parametrize("name", sorted(SMALL))
def test_compaction_matches_oracle(name):
    wl, x = make(name)
    k_out, v_out, kept, klen = run_compact(wl, x)
    h = host(x)
    K, KL = to_np(kept), to_np(klen)
    ko, vo = bf16_bits(k_out), bf16_bits(v_out)
    for b, n in enumerate(h["lens"]):
        L = int(n) - wl.window
        for g in range(wl.num_kv_heads):
            kl = int(KL[b, g])
            idx = K[b, g, :kl]
            if L <= wl.budget:
                assert kl == n and (idx == np.arange(n)).all()
            else:
                assert kl == wl.budget + wl.window
                assert (idx[wl.budget:] == np.arange(L, n)).all()
                pooled = oracle.maxpool1d(oracle_votes(h, wl, b, g), wl.pool_kernel)
                check_selection(idx[:wl.budget], pooled, wl.budget, f"{name} b{b} g{g}")
            assert (K[b, g, kl:] == -1).all()
            assert (ko[b, g, :kl] == h["k"][b, g, idx]).all()
            assert (vo[b, g, :kl] == h["v"][b, g, idx]).all()


@pytest.mark.parametrize("name", ["d128_g4_w32", "d64_g2_w8", "d128_g32_w8"])
def test_decode_over_compacted_cache(name):
    wl, x = make(name)
    k_out, v_out, kept, klen = run_compact(wl, x)
    KL = to_np(klen)
    B, H, C, D = wl.batch, wl.num_kv_heads, wl.out_capacity, wl.head_dim
    L = se.dense_layout(H, C, D)
    MP = C // 16
    pt = (torch.arange(B, device=DEV)[:, None] * (H * MP) + torch.arange(MP, device=DEV)[None]).to(torch.int32)
    P = se.decode_params(B, wl.num_q_heads, MP, MP, wl.scale)
    ws = workspace(se.se_sparse_decode_workspace_size(L, P))
    out = torch.empty((B, wl.num_q_heads, D), dtype=torch.float32, device=DEV)
    base = torch.from_numpy(KL[:, 0].astype(np.int64)).to(DEV)
    for s in range(wl.decode_steps):
        rows = base + s
        bi = torch.arange(B, device=DEV)
        k_out[bi, :, rows] = x["k_steps"][s]
        v_out[bi, :, rows] = x["v_steps"][s]
        lens = (rows + 1).to(torch.int32)
        call_twice(lambda: se.se_sparse_decode(L, P, x["q_steps"][s], k_out, v_out, pt, None, lens, out, None, ws), ws,
                   [out], f"{name} step {s}")
        ko, vo, q = bf16_bits(k_out), bf16_bits(v_out), bf16_bits(x["q_steps"][s])
        o = to_np(out)
        for b in range(B):
            ref = oracle.decode_over_rows(q[b], ko[b], vo[b], int(lens[b]), wl.group, wl.scale)
            check_attention(o[b], ref, 8.0, f"{name} step {s} b{b}")


def test_longest_prompt_selection_and_copies():
    """The longest prompt the library takes (a 65,536-token prefix before the
    32-token window): the kept positions of one (request, KV head) against
    the oracle's pooled votes, and the kept rows copied bit for bit."""
    n = 65536 + 32
    wl = SnapKVWorkload("s_long", 1, 4, 1, 128, n, 32, 7, 2048, 1, seed=38)
    x = make_snapkv_inputs(wl, DEV, prompt_lens=[n])
    announce(f"snapkv longest prompt seed {wl.seed}")
    p = params(wl)
    ws = workspace(se.se_snapkv_workspace_size(p))
    kcap = wl.budget + wl.window
    k_out = torch.zeros((1, 1, wl.out_capacity, wl.head_dim), dtype=torch.bfloat16, device=DEV)
    v_out = torch.zeros_like(k_out)
    kept = torch.full((1, 1, kcap), 777, dtype=torch.int32, device=DEV)
    klen = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    call_twice(lambda: se.se_snapkv_compact(p, x["q_win"], x["k"], x["v"], x["prompt_lens"], k_out, v_out, kept, klen,
                                            ws), ws, [k_out, v_out, kept, klen], "longest prompt")
    n, Lp = wl.prompt, wl.prompt - wl.window
    K = to_np(kept)[0, 0]
    assert int(to_np(klen)[0, 0]) == kcap
    assert (K[wl.budget:] == np.arange(Lp, n)).all()
    h = host(x)
    S = oracle_votes(h, wl, 0, 0)
    check_selection(K[:wl.budget], oracle.maxpool1d(S, wl.pool_kernel), wl.budget, "longest prompt")
    for src, dst in ((x["k"], k_out), (x["v"], v_out)):
        want = src[0, 0, torch.from_numpy(K).long().to(DEV)]
        assert torch.equal(want.view(torch.int16), dst[0, 0, :kcap].view(torch.int16))
