"""Parity at the full workload sizes, in the launch configuration the
benchmark times (auto split count, max head aggregation, fused last-page
refresh).  The whole batch runs on the GPU; the oracle recomputes sampled
(request, KV head) units one by one, and properties that hold at any size
(counts, ordering, finiteness, bitwise copies) are checked on every unit.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_long_amd as se
from synth import (H2O_32K, MLA_RAGGED, PRUNE_32K, PYRAMID_32K, QWEN3_4B_32K, QWEN3_30B_128K, SNAPKV_32K, make_quest_inputs,
                   make_snapkv_inputs, bf16_bits)
from gpu_util import DEV, announce, build_summaries, check_attention, check_selection, layout_for, to_np, workspace

pytestmark = pytest.mark.gpu

QUEST_FULL = {w.name: w for w in (QWEN3_4B_32K, QWEN3_30B_128K, MLA_RAGGED)}


def _unit_rows(pages, phys, g):
    """bf16 bits [P, 16, D] of KV head g on the given physical pages."""
    idx = torch.from_numpy(np.asarray(phys, dtype=np.int64)).to(pages.device)
    return bf16_bits(pages.index_select(0, idx)[:, g])


def _sample_units(wl, lens, count=3):
    rng = np.random.default_rng(wl.seed + 5)
    units = {(int(np.argmin(lens)), 0), (int(np.argmax(lens)), wl.num_kv_heads - 1)}
    while len(units) < count:
        units.add((int(rng.integers(wl.batch)), int(rng.integers(wl.num_kv_heads))))
    return sorted(units)


@pytest.mark.parametrize("name", sorted(QUEST_FULL))
def test_quest_full_size_sampled_units(name):
    wl = QUEST_FULL[name]
    announce(f"full-size quest {name} seed {wl.seed}")
    x = make_quest_inputs(wl, DEV, poison_tail=True)
    summ = build_summaries(x, wl)
    L = layout_for(wl)
    P = se.decode_params(wl.batch, wl.num_q_heads, wl.max_pages, wl.topk, wl.scale, 0, 1, 0)
    ws = workspace(se.se_sparse_decode_workspace_size(L, P))
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32, device=DEV)
    sel = torch.empty((wl.batch, wl.num_kv_heads, wl.topk), dtype=torch.int32, device=DEV)
    se.se_sparse_decode(L, P, x["q"], x["k_pages"], x["v_pages"], x["page_table"], summ, x["seq_lens"], out, sel, ws)
    torch.cuda.synchronize()

    lens = to_np(x["seq_lens"]).astype(np.int64)
    pt = to_np(x["page_table"])
    o = to_np(out)
    S = to_np(sel)
    G = wl.group
    # properties on every unit
    assert np.isfinite(o).all()
    for b, n in enumerate(lens):
        k = min(wl.topk, -(-int(n) // 16))
        for g in range(wl.num_kv_heads):
            ids = S[b, g, :k]
            assert (np.diff(ids) > 0).all() and ids[0] >= 0 and ids[-1] < -(-int(n) // 16)
            assert (S[b, g, k:] == -1).all()
    # the oracle on sampled units
    q = bf16_bits(x["q"])
    for b, g in _sample_units(wl, lens):
        n = int(lens[b])
        Pb = -(-n // 16)
        announce(f"{name} unit b{b} g{g} n{n}")
        kbits = _unit_rows(x["k_pages"], pt[b, :Pb], g)
        kp = oracle.gather_unit_pages(kbits[:, None], np.arange(Pb), 0, n)
        mins, maxs = oracle.unit_summaries(kp, n)
        gs = bf16_bits(summ.index_select(0, torch.from_numpy(pt[b, :Pb].astype(np.int64)).to(DEV))[:, g])
        assert (oracle.bf16_to_f64(gs[:, 0]) == mins).all() and (oracle.bf16_to_f64(gs[:, 1]) == maxs).all()
        qf = oracle.bf16_to_f64(q[b, g * G:(g + 1) * G])
        A = oracle.unit_kv_head_score(oracle.unit_page_bounds(qf, mins, maxs, wl.scale))
        k = min(wl.topk, Pb)
        check_selection(S[b, g], A, wl.topk, f"{name} b{b} g{g}")
        chosen = S[b, g, :k].astype(np.int64)
        keys = oracle.unit_selected_tokens(kp, chosen, n)
        if wl.v_is_k_prefix:
            vals = keys[:, :wl.head_dim_v]
        else:
            vbits = _unit_rows(x["v_pages"], pt[b, :Pb], g)
            vals = oracle.unit_selected_tokens(oracle.gather_unit_pages(vbits[:, None], np.arange(Pb), 0, n), chosen, n)
        ref = oracle.unit_attention(qf, keys, vals, wl.scale)
        check_attention(o[b, g * G:(g + 1) * G], ref, float(np.abs(vals).max()), f"{name} b{b} g{g}")


def test_snapkv_full_size_sampled_units():
    wl = SNAPKV_32K
    announce(f"full-size snapkv {wl.name} seed {wl.seed}")
    x = make_snapkv_inputs(wl, DEV)
    p = se.snapkv_params(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.prompt, wl.window,
                         wl.pool_kernel, wl.budget, wl.out_capacity, wl.scale)
    ws = workspace(se.se_snapkv_workspace_size(p))
    B, H, C, D = wl.batch, wl.num_kv_heads, wl.out_capacity, wl.head_dim
    k_out = torch.zeros((B, H, C, D), dtype=torch.bfloat16, device=DEV)
    v_out = torch.zeros((B, H, C, D), dtype=torch.bfloat16, device=DEV)
    kept = torch.full((B, H, wl.budget + wl.window), 777, dtype=torch.int32, device=DEV)
    klen = torch.zeros((B, H), dtype=torch.int32, device=DEV)
    se.se_snapkv_compact(p, x["q_win"], x["k"], x["v"], x["prompt_lens"], k_out, v_out, kept, klen, ws)
    torch.cuda.synchronize()
    n = wl.prompt
    Lp = n - wl.window
    K, KL = to_np(kept), to_np(klen)
    # properties on every unit: counts, the window tail, ascending ids, bitwise copies
    assert (KL == wl.budget + wl.window).all()
    assert (K[..., wl.budget:] == np.arange(Lp, n)).all()
    assert (np.diff(K, axis=-1) > 0).all()
    idx = kept.long()
    for src, dst in ((x["k"], k_out), (x["v"], v_out)):
        gathered = torch.gather(src, 2, idx[..., None].expand(-1, -1, -1, D))
        assert torch.equal(gathered.view(torch.int16), dst[:, :, :wl.budget + wl.window].view(torch.int16))
        assert not dst[:, :, wl.budget + wl.window:].view(torch.int16).any()
    # votes, pool and selection on sampled units
    qb = bf16_bits(x["q_win"])
    G = wl.group
    for b, g in ((0, 0), (7, 3), (B - 1, H - 1)):
        announce(f"snapkv unit b{b} g{g}")
        keys = oracle.bf16_to_f64(bf16_bits(x["k"][b, g]))
        Sv, _, _ = oracle.snapkv_unit_votes(oracle.bf16_to_f64(qb[b, g * G:(g + 1) * G]), keys, n, wl.scale)
        pooled = oracle.maxpool1d(Sv, wl.pool_kernel)
        check_selection(K[b, g, :wl.budget], pooled, wl.budget, f"snapkv b{b} g{g}")

    # decode over the compacted cache: the 64 steps the workload runs, oracle on steps 0 and 63
    Ld = se.dense_layout(H, C, D)
    MP = C // 16
    pt = (torch.arange(B, device=DEV)[:, None] * (H * MP) + torch.arange(MP, device=DEV)[None]).to(torch.int32)
    Pd = se.decode_params(B, wl.num_q_heads, MP, MP, wl.scale)
    wsd = workspace(se.se_sparse_decode_workspace_size(Ld, Pd))
    out = torch.empty((B, wl.num_q_heads, D), dtype=torch.float32, device=DEV)
    base = klen[:, 0].long()
    bi = torch.arange(B, device=DEV)
    for s in range(wl.decode_steps):
        rows = base + s
        k_out[bi, :, rows] = x["k_steps"][s]
        v_out[bi, :, rows] = x["v_steps"][s]
        lens = (rows + 1).to(torch.int32)
        se.se_sparse_decode(Ld, Pd, x["q_steps"][s], k_out, v_out, pt, None, lens, out, None, wsd)
        if s in (0, wl.decode_steps - 1):
            torch.cuda.synchronize()
            o = to_np(out)
            qs = bf16_bits(x["q_steps"][s])
            for b in (0, B - 1):
                ko, vo = bf16_bits(k_out[b]), bf16_bits(v_out[b])
                ref = oracle.decode_over_rows(qs[b], ko, vo, int(lens[b]), G, wl.scale)
                check_attention(o[b], ref, float(np.abs(oracle.bf16_to_f64(vo)).max()), f"snapkv step {s} b{b}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["h2o", "prune", "pyramid_layer0", "pyramid_layer3"])
def test_eviction_family_full_size_sampled_units(name):
    """The H2O, prefix-pruning and PyramidKV legs at the size the bench runs
    (PyramidKV: its first and last layers' budgets): counts, forced tokens
    and bitwise copies on every unit, votes and selection on sampled units
    against the oracle."""
    if name.startswith("pyramid"):
        budgets = se.se_pyramid_budgets(PYRAMID_32K.layers, PYRAMID_32K.budget, *PYRAMID_32K.layer_ratios)
        assert budgets == oracle.pyramid_budgets(PYRAMID_32K.layers, PYRAMID_32K.budget, *PYRAMID_32K.layer_ratios)
        wl = PYRAMID_32K.resized(budget=budgets[int(name[-1])], layers=1)
    else:
        wl = {"h2o": H2O_32K, "prune": PRUNE_32K}[name]
    announce(f"full-size eviction {wl.name} seed {wl.seed}")
    x = make_snapkv_inputs(wl, DEV, with_decode=False)
    iv = wl.interval if wl.interval[1] else None
    kcap = oracle.eviction_kept_capacity(wl.prompt, wl.window, wl.budget, wl.sink, wl.recent, iv)
    p = se.snapkv_params(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.prompt, wl.window,
                         wl.pool_kernel, wl.budget, (kcap + 15) // 16 * 16, wl.scale, sink=wl.sink,
                         recent=wl.recent, interval=wl.interval)
    assert se.se_snapkv_kept_capacity(p) == kcap
    ws = workspace(se.se_snapkv_workspace_size(p))
    B, H, C, D = wl.batch, wl.num_kv_heads, p.out_capacity, wl.head_dim
    k_out = torch.zeros((B, H, C, D), dtype=torch.bfloat16, device=DEV)
    v_out = torch.zeros((B, H, C, D), dtype=torch.bfloat16, device=DEV)
    kept = torch.full((B, H, kcap), 777, dtype=torch.int32, device=DEV)
    klen = torch.zeros((B, H), dtype=torch.int32, device=DEV)
    se.se_snapkv_compact(p, x["q_win"], x["k"], x["v"], x["prompt_lens"], k_out, v_out, kept, klen, ws)
    torch.cuda.synchronize()
    n = wl.prompt
    lo, hi = oracle.eviction_candidates(n, wl.window, wl.sink, wl.recent, iv)
    R = wl.budget
    K, KL = to_np(kept), to_np(klen)
    assert hi - lo > R and (KL == lo + R + n - hi).all() and kcap == lo + R + n - hi
    assert (K[..., :lo] == np.arange(lo)).all() and (K[..., lo + R:] == np.arange(hi, n)).all()
    assert (np.diff(K, axis=-1) > 0).all()
    idx = kept.long()
    for src, dst in ((x["k"], k_out), (x["v"], v_out)):
        gathered = torch.gather(src, 2, idx[..., None].expand(-1, -1, -1, D))
        assert torch.equal(gathered.view(torch.int16), dst[:, :, :kcap].view(torch.int16))
    qb = bf16_bits(x["q_win"])
    G = wl.group
    for b, g in ((0, 0), (B - 1, H - 1)):
        announce(f"{wl.name} unit b{b} g{g}")
        keys = oracle.bf16_to_f64(bf16_bits(x["k"][b, g]))
        Sv, _, _ = oracle.snapkv_unit_votes(oracle.bf16_to_f64(qb[b, g * G:(g + 1) * G]), keys, n, wl.scale)
        pooled = oracle.maxpool1d(Sv, wl.pool_kernel)
        check_selection(K[b, g, lo:lo + R] - lo, pooled[lo:hi], R, f"{wl.name} b{b} g{g}")
