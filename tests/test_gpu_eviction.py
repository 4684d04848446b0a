"""GPU parity of the eviction family around SnapKV's scores, through the C
ABI: sink and recent tokens beside the selected budget, H2O's 128-token
scoring window with a recent share and no pooling, prefix-cache pruning inside
a history interval, PyramidKV's per-layer budgets, and re-eviction of a
compacted cache after decode steps (original positions composed)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_long_amd as se
from synth import SnapKVWorkload, make_snapkv_inputs, bf16_bits
from gpu_util import call_twice, DEV, announce, check_attention, check_selection, to_np, workspace

pytestmark = pytest.mark.gpu

# name: (workload, prompt lengths, sink, recent, interval)
CASES = {
    # Table 9's SnapKV shape: 16-token window, sink 16, recent 64
    "snapkv_sink16_recent64": (SnapKVWorkload("e_snap", 4, 8, 2, 128, 1000, 16, 7, 100, 0, seed=41),
                               [1000, 700, 181, 150], 16, 64, None),
    # H2O: 128-token scoring window, no pooling, recent ratio 0.5 of a 400-token total
    "h2o_w128_g4": (SnapKVWorkload("e_h2o", 3, 8, 2, 128, 1500, 128, 1, 200, 0, seed=42),
                    [1500, 900, 401], 0, 200, None),
    "h2o_w128_g8_d64": (SnapKVWorkload("e_h2o64", 2, 8, 1, 64, 1200, 128, 1, 150, 0, seed=43),
                        [1200, 640], 0, 150, None),
    # enough (request, KV head) units that each key-tile walker of the
    # row-groups-as-waves passes takes several tiles (one to six, odd and even
    # counts), so the loop that keeps the next tile in flight runs every branch
    "h2o_w128_multitile": (SnapKVWorkload("e_h2o_mt", 4, 32, 8, 128, 3000, 128, 1, 300, 0, seed=49),
                           [3000, 2500, 1000, 520], 0, 300, None),
    # edge lengths: empty, shorter than the window, exactly the window, exactly
    # sink + recent (nothing to choose from), one candidate past the budget
    "edges_sink_recent": (SnapKVWorkload("e_edge", 7, 8, 2, 128, 400, 16, 5, 30, 0, seed=47),
                          [0, 9, 16, 48, 78, 79, 400], 8, 40, None),
    "edges_interval": (SnapKVWorkload("e_edge2", 6, 4, 2, 64, 300, 8, 3, 20, 0, seed=48),
                       [0, 7, 60, 121, 150, 300], 2, 0, (100, 141)),
    # prefix-cache pruning: only positions 200..699 may go
    "prune_200_700": (SnapKVWorkload("e_prune", 4, 8, 2, 128, 1000, 32, 7, 60, 0, seed=44),
                      [1000, 650, 260, 100], 0, 0, (200, 700)),
    # sink beyond the interval start, recent beyond its end
    "prune_sink_recent": (SnapKVWorkload("e_prune2", 2, 4, 1, 128, 900, 16, 5, 40, 0, seed=45),
                          [900, 500], 120, 300, (50, 800)),
}


def params(wl, sink, recent, interval, out_capacity=None, max_len=None):
    N = wl.prompt if max_len is None else max_len
    kcap = oracle.eviction_kept_capacity(N, wl.window, wl.budget, sink, recent, interval)
    return se.snapkv_params(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, N, wl.window,
                            wl.pool_kernel, wl.budget, out_capacity or -(-kcap // 16) * 16, wl.scale,
                            sink=sink, recent=recent, interval=interval or (0, 0)), kcap


def run_evict(p, kcap, q_win, k, v, lens, positions=None):
    B, H, D = p.batch, p.num_kv_heads, p.head_dim
    ws = workspace(se.se_snapkv_workspace_size(p))
    assert se.se_snapkv_kept_capacity(p) == kcap
    k_out = torch.zeros((B, H, p.out_capacity, D), dtype=torch.bfloat16, device=DEV)
    v_out = torch.zeros((B, H, p.out_capacity, D), dtype=torch.bfloat16, device=DEV)
    kept = torch.full((B, H, kcap), 777, dtype=torch.int32, device=DEV)
    klen = torch.zeros((B, H), dtype=torch.int32, device=DEV)
    if positions is None:
        call = lambda: se.se_snapkv_compact(p, q_win, k, v, lens, k_out, v_out, kept, klen, ws)
    else:
        call = lambda: se.se_snapkv_recompact(p, q_win, k, v, lens, positions, k_out, v_out, kept, klen, ws)
    call_twice(call, ws, [k_out, v_out, kept, klen], "eviction")
    return k_out, v_out, kept, klen


def check_unit(rows, kl, n, wl, sink, recent, interval, qw_bits, k_bits, what):
    """rows: the GPU's kept cache rows of one (b, g); checks forced rows exactly
    and the chosen candidates by the gap rule on the oracle's pooled votes."""
    lo, hi = oracle.eviction_candidates(n, wl.window, sink, recent, interval)
    R = wl.budget
    if hi - lo <= R:
        assert kl == n and (rows == np.arange(n)).all(), what
        return
    assert kl == lo + R + (n - hi), what
    assert (rows[:lo] == np.arange(lo)).all(), f"{what}: forced head"
    assert (rows[lo + R:kl] == np.arange(hi, n)).all(), f"{what}: forced tail"
    S, _, _ = oracle.snapkv_unit_votes(oracle.bf16_to_f64(qw_bits), oracle.bf16_to_f64(k_bits), n, wl.scale)
    pooled = oracle.maxpool1d(S, wl.pool_kernel)
    check_selection(rows[lo:lo + R] - lo, pooled[lo:hi], R, what)


@pytest.mark.parametrize("name", sorted(CASES))
def test_eviction_family_matches_oracle(name):
    wl, lens, sink, recent, iv = CASES[name]
    announce(f"eviction case {name} seed {wl.seed} lens {lens}")
    x = make_snapkv_inputs(wl, DEV, prompt_lens=lens, with_decode=False)
    p, kcap = params(wl, sink, recent, iv)
    k_out, v_out, kept, klen = run_evict(p, kcap, x["q_win"], x["k"], x["v"], x["prompt_lens"])
    K, KL = to_np(kept), to_np(klen)
    qb, kb, vb = bf16_bits(x["q_win"]), bf16_bits(x["k"]), bf16_bits(x["v"])
    ko, vo = bf16_bits(k_out), bf16_bits(v_out)
    G = wl.group
    for b, n in enumerate(lens):
        for g in range(wl.num_kv_heads):
            kl = int(KL[b, g])
            rows = K[b, g, :kl]
            assert (K[b, g, kl:] == -1).all()
            check_unit(rows, kl, n, wl, sink, recent, iv, qb[b, g * G:(g + 1) * G], kb[b, g], f"{name} b{b} g{g}")
            assert (ko[b, g, :kl] == kb[b, g, rows]).all() and (vo[b, g, :kl] == vb[b, g, rows]).all()
            assert not ko[b, g, kl:].any()


@pytest.mark.parametrize("name", ["h2o_w128_g4", "h2o_w128_multitile"])
def test_h2o_votes_match_oracle(name):
    """The 128-row window's votes themselves (four row groups of 128 rows)."""
    wl, lens, sink, recent, iv = CASES[name]
    announce(f"h2o votes case {name} seed {wl.seed} lens {lens}")
    x = make_snapkv_inputs(wl, DEV, prompt_lens=lens, with_decode=False)
    p, _ = params(wl, sink, recent, iv)
    ws = workspace(se.se_snapkv_workspace_size(p))
    votes = torch.full((wl.batch, wl.num_kv_heads, wl.prompt), float("nan"), device=DEV)
    call_twice(lambda: se.se_snapkv_votes(p, x["q_win"], x["k"], x["prompt_lens"], votes, ws), ws, [votes], "h2o votes")
    V = to_np(votes)
    qb, kb = bf16_bits(x["q_win"]), bf16_bits(x["k"])
    G = wl.group
    for b, n in enumerate(lens):
        for g in range(wl.num_kv_heads):
            L = n - wl.window
            S, _, _ = oracle.snapkv_unit_votes(oracle.bf16_to_f64(qb[b, g * G:(g + 1) * G]),
                                               oracle.bf16_to_f64(kb[b, g]), n, wl.scale)
            err = np.abs(V[b, g, :L] - S)
            tol = 2e-4 * S + 1e-6 * S.max()
            assert (err <= tol).all(), f"b{b} g{g}: worst {np.max(err / tol):.3f} of tolerance"


def test_pyramid_layers_match_oracle():
    """PyramidKV: one eviction per layer with the layer's budget from the
    library's schedule (Table 8's sink 64 / recent 512 scaled down with the
    prompt), each layer its own window queries and cache."""
    layers = 4
    budgets = se.se_pyramid_budgets(layers, 96, 0.6, 0.01)
    assert budgets == oracle.pyramid_budgets(layers, 96, 0.6, 0.01)
    for layer, R in enumerate(budgets):
        wl = SnapKVWorkload(f"e_pyr{layer}", 2, 8, 2, 128, 1100, 32, 7, R, 0, seed=50 + layer)
        lens = [1100, 420]
        announce(f"pyramid layer {layer} budget {R} seed {wl.seed}")
        x = make_snapkv_inputs(wl, DEV, prompt_lens=lens, with_decode=False)
        p, kcap = params(wl, 8, 64, None)
        k_out, v_out, kept, klen = run_evict(p, kcap, x["q_win"], x["k"], x["v"], x["prompt_lens"])
        K, KL = to_np(kept), to_np(klen)
        qb, kb = bf16_bits(x["q_win"]), bf16_bits(x["k"])
        for b, n in enumerate(lens):
            for g in range(2):
                kl = int(KL[b, g])
                check_unit(K[b, g, :kl], kl, n, wl, 8, 64, None, qb[b, 4 * g:4 * g + 4], kb[b, g],
                           f"layer {layer} b{b} g{g}")


# (window, pool, decode steps, sink, recent, budget of the second eviction, first interval)
REEVICT = {
    "snapkv": (16, 7, 48, 4, 32, 50, None),
    "snapkv_interval": (16, 7, 48, 4, 32, 50, (40, 600)),
    # H2O's shape: a 128-query window (four row groups), no pooling, the recent share as forced tokens
    "h2o": (128, 1, 136, 0, 150, 90, None),
}


@pytest.mark.parametrize("case", sorted(REEVICT))
def test_reeviction_after_decode_steps(case):
    """Prefill eviction, decode steps appended to the retained cache, then a
    second eviction over that cache with the last W decode queries as the
    window; kept_idx must report original positions, and a decode step over
    the re-evicted cache must match the oracle."""
    W_, pool, steps, sink, recent, budget2, first_interval = REEVICT[case]
    wl = SnapKVWorkload("e_re", 3, 8, 2, 128, 900, W_, pool, 120, steps, seed=46)
    lens = [900, 610, 300]
    announce(f"re-eviction {case} seed {wl.seed} lens {lens}")
    x = make_snapkv_inputs(wl, DEV, prompt_lens=lens)
    B, H, D, G, S, W = wl.batch, wl.num_kv_heads, wl.head_dim, wl.group, wl.decode_steps, wl.window
    p1, kcap1 = params(wl, sink, recent, first_interval)
    C1 = -(-(kcap1 + S) // 16) * 16
    p1.out_capacity = C1
    k1, v1, kept1, klen1 = run_evict(p1, kcap1, x["q_win"], x["k"], x["v"], x["prompt_lens"])
    KL1 = to_np(klen1)
    assert (KL1 == KL1[:, :1]).all()
    # decode steps: append k, v at rows kept_len + s (the engine's append)
    base = klen1[:, 0].long()
    bi = torch.arange(B, device=DEV)
    for s in range(S):
        k1[bi, :, base + s] = x["k_steps"][s]
        v1[bi, :, base + s] = x["v_steps"][s]
    cache_lens = (base + S).to(torch.int32)
    positions = torch.full((B, H, C1), -1, dtype=torch.int32, device=DEV)
    positions[:, :, :kcap1] = kept1
    for b in range(B):
        kl = int(KL1[b, 0])
        positions[b, :, kl:kl + S] = torch.arange(lens[b], lens[b] + S, dtype=torch.int32, device=DEV)
    q_win2 = x["q_steps"][S - W:].permute(1, 2, 0, 3).contiguous()  # [B, Hq, W, D]
    wl2 = wl.resized(budget=budget2)
    p2, kcap2 = params(wl2, sink, recent, None, max_len=C1)
    k2, v2, kept2, klen2 = run_evict(p2, kcap2, q_win2, k1, v1, cache_lens, positions=positions)

    # the oracle's re-eviction over the same cache rows and positions
    ok2, ov2, okept2, oklen2, _ = oracle.snapkv_compact(
        bf16_bits(q_win2), bf16_bits(k1), bf16_bits(v1), to_np(cache_lens), G, wl.scale, W, wl.pool_kernel,
        wl2.budget, p2.out_capacity, sink=sink, recent=recent, positions=to_np(positions))
    K2, KL2, pos = to_np(kept2), to_np(klen2), to_np(positions)
    qb, kb1, vb1 = bf16_bits(q_win2), bf16_bits(k1), bf16_bits(v1)
    ko2, vo2 = bf16_bits(k2), bf16_bits(v2)
    for b in range(B):
        n = int(cache_lens[b])
        for g in range(H):
            kl = int(KL2[b, g])
            assert kl == oklen2[b, g]
            got = K2[b, g, :kl]
            assert (K2[b, g, kl:] == -1).all()
            # original positions are increasing, so they map back to cache rows
            rows = np.searchsorted(pos[b, g, :n], got)
            assert (pos[b, g, rows] == got).all(), "kept_idx is not a position of the cache"
            check_unit(rows, kl, n, wl2, sink, recent, None, qb[b, g * G:(g + 1) * G], kb1[b, g],
                       f"re-evict b{b} g{g}")
            assert (ko2[b, g, :kl] == kb1[b, g, rows]).all() and (vo2[b, g, :kl] == vb1[b, g, rows]).all()
            # forced rows are exact, so their positions equal the oracle's
            lo, hi = oracle.eviction_candidates(n, W, sink, recent)
            if hi - lo > wl2.budget:
                assert (got[:lo] == okept2[b, g, :lo]).all() and (got[lo + wl2.budget:] == okept2[b, g, lo + wl2.budget:kl]).all()

    # one decode step over the re-evicted cache
    C2 = p2.out_capacity
    MP = C2 // 16
    Ld = se.dense_layout(H, C2, D)
    Pd = se.decode_params(B, wl.num_q_heads, MP, MP, wl.scale)
    wsd = workspace(se.se_sparse_decode_workspace_size(Ld, Pd))
    pt = (torch.arange(B, device=DEV)[:, None] * (H * MP) + torch.arange(MP, device=DEV)[None]).to(torch.int32)
    out = torch.empty((B, wl.num_q_heads, D), dtype=torch.float32, device=DEV)
    dl = klen2[:, 0].to(torch.int32)
    call_twice(lambda: se.se_sparse_decode(Ld, Pd, x["q_steps"][S - 1], k2, v2, pt, None, dl, out, None, wsd), wsd,
               [out], "decode after re-eviction")
    o, qs = to_np(out), bf16_bits(x["q_steps"][S - 1])
    for b in range(B):
        ref = oracle.decode_over_rows(qs[b], ko2[b], vo2[b], int(dl[b]), G, wl.scale)
        check_attention(o[b], ref, float(np.abs(oracle.bf16_to_f64(vo2[b])).max()), f"decode after re-evict b{b}")


@pytest.mark.parametrize("sink,recent,interval", [(5, 40, None), (0, 0, (60, 250)), (30, 70, (10, 200)),
                                                  (0, 120, None)])
def test_select_and_compact_exact_on_given_votes(sink, recent, interval):
    """se_maxpool1d, se_snapkv_select and se_compact one by one on integer-valued
    votes (ties on purpose): the pooled values and the kept positions equal the
    oracle's exactly (the lower position wins a tie), and the copies are bitwise."""
    wl = SnapKVWorkload("e_sel", 3, 8, 2, 128, 300, 16, 5, 40, 0, seed=49)
    lens = [300, 171, 90]
    x = make_snapkv_inputs(wl, DEV, prompt_lens=lens, with_decode=False)
    p, kcap = params(wl, sink, recent, interval)
    rng = np.random.default_rng(49)
    votes = rng.integers(0, 6, (wl.batch, wl.num_kv_heads, wl.prompt)).astype(np.float32) / 4
    pooled = torch.full((wl.batch, wl.num_kv_heads, wl.prompt), float("nan"), device=DEV)
    se.se_maxpool1d(p, torch.from_numpy(votes).to(DEV), x["prompt_lens"], pooled)
    kept = torch.full((wl.batch, wl.num_kv_heads, kcap), 777, dtype=torch.int32, device=DEV)
    klen = torch.zeros((wl.batch, wl.num_kv_heads), dtype=torch.int32, device=DEV)
    se.se_snapkv_select(p, pooled, x["prompt_lens"], kept, klen)
    k_out = torch.zeros((wl.batch, wl.num_kv_heads, p.out_capacity, wl.head_dim), dtype=torch.bfloat16, device=DEV)
    v_out = torch.zeros_like(k_out)
    se.se_compact(p, x["k"], x["v"], kept, klen, k_out, v_out)
    torch.cuda.synchronize()
    Pg, K, KL = to_np(pooled), to_np(kept), to_np(klen)
    kb, vb, ko, vo = bf16_bits(x["k"]), bf16_bits(x["v"]), bf16_bits(k_out), bf16_bits(v_out)
    for b, n in enumerate(lens):
        L = n - wl.window
        for g in range(wl.num_kv_heads):
            want_pool = oracle.maxpool1d(votes[b, g, :L].astype(np.float64), wl.pool_kernel)
            assert (Pg[b, g, :L] == want_pool).all()
            keep = oracle.eviction_unit_keep(want_pool, n, wl.window, wl.budget, sink, recent, interval)
            assert KL[b, g] == len(keep), (b, g)
            assert (K[b, g, :len(keep)] == keep).all() and (K[b, g, len(keep):] == -1).all(), (b, g)
            assert (ko[b, g, :len(keep)] == kb[b, g, keep]).all() and (vo[b, g, :len(keep)] == vb[b, g, keep]).all()
