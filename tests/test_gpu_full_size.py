"""Parity at the full workload sizes, in the launch configuration the
benchmark times (auto split count, max head aggregation, fused last-page
refresh).  The whole batch runs on the GPU; the oracle recomputes EVERY
(request, KV head) unit -- summaries bitwise, selection by the gap rule,
attention on the GPU's selection -- in worker processes (tests/oracle_pool.py,
CPU only), and properties that hold at any size (counts, ordering,
finiteness, bitwise copies) are checked on every unit as well.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_long_amd as se
from synth import (H2O_32K, MLA_RAGGED, PRUNE_32K, PYRAMID_32K, QWEN3_4B_32K, QWEN3_30B_128K, SNAPKV_32K, make_quest_inputs,
                   make_snapkv_inputs, bf16_bits)
from gpu_util import (DEV, announce, build_summaries, call_twice, check_attention, check_selection, layout_for, to_np,
                      workspace)
import oracle_pool

pytestmark = pytest.mark.gpu

QUEST_FULL = {w.name: w for w in (QWEN3_4B_32K, QWEN3_30B_128K, MLA_RAGGED)}


def _unit_rows(pages, phys, g):
    """bf16 bits [P, 16, D] of KV head g on the given physical pages."""
    idx = torch.from_numpy(np.asarray(phys, dtype=np.int64)).to(pages.device)
    return bf16_bits(pages.index_select(0, idx)[:, g])


@pytest.mark.parametrize("name", sorted(QUEST_FULL))
def test_quest_full_size_every_unit(name):
    wl = QUEST_FULL[name]
    announce(f"full-size quest {name} seed {wl.seed}")
    x = make_quest_inputs(wl, DEV, poison_tail=True)
    summ = build_summaries(x, wl)
    L = layout_for(wl)
    P = se.decode_params(wl.batch, wl.num_q_heads, wl.max_pages, wl.topk, wl.scale, 0, 1, 0)
    ws = workspace(se.se_sparse_decode_workspace_size(L, P))
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32, device=DEV)
    sel = torch.empty((wl.batch, wl.num_kv_heads, wl.topk), dtype=torch.int32, device=DEV)
    call_twice(lambda: se.se_sparse_decode(L, P, x["q"], x["k_pages"], x["v_pages"], x["page_table"], summ,
                                           x["seq_lens"], out, sel, ws), ws, [out, sel], f"full-size {name}")

    lens = to_np(x["seq_lens"]).astype(np.int64)
    pt = to_np(x["page_table"])
    o = to_np(out)
    S = to_np(sel)
    G = wl.group
    assert np.isfinite(o).all()
    q = bf16_bits(x["q"])
    units = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]

    def jobs():
        for b, g in units:
            n = int(lens[b])
            Pb = -(-n // 16)
            k = min(wl.topk, Pb)
            chosen = S[b, g, :k].astype(np.int64)
            assert (np.diff(chosen) > 0).all() and chosen[0] >= 0 and chosen[-1] < Pb, f"b{b} g{g}: ids"
            assert (S[b, g, k:] == -1).all(), f"b{b} g{g}: padding"
            kbits = _unit_rows(x["k_pages"], pt[b, :Pb], g)
            vbits = None if wl.v_is_k_prefix else _unit_rows(x["v_pages"], pt[b, chosen], g)
            yield (b, g), (kbits, vbits, q[b, g * G:(g + 1) * G], n, wl.scale, chosen, wl.head_dim_v,
                           wl.v_is_k_prefix)

    checked = 0
    with oracle_pool.pool() as ex:
        for (b, g), (mins, maxs, A, ref, vmax) in oracle_pool.map_bounded(ex, oracle_pool.quest_unit, jobs()):
            n = int(lens[b])
            Pb = -(-n // 16)
            gs = bf16_bits(summ.index_select(0, torch.from_numpy(pt[b, :Pb].astype(np.int64)).to(DEV))[:, g])
            assert (oracle.bf16_to_f64(gs[:, 0]) == mins).all() and (oracle.bf16_to_f64(gs[:, 1]) == maxs).all(), \
                f"{name} b{b} g{g}: summaries"
            check_selection(S[b, g], A, wl.topk, f"{name} b{b} g{g}")
            check_attention(o[b, g * G:(g + 1) * G], ref, vmax, f"{name} b{b} g{g}")
            checked += 1
    assert checked == len(units)
    announce(f"{name}: {checked} units match the oracle")


def test_snapkv_full_size_every_unit():
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
    call_twice(lambda: se.se_snapkv_compact(p, x["q_win"], x["k"], x["v"], x["prompt_lens"], k_out, v_out, kept, klen,
                                            ws), ws, [k_out, v_out, kept, klen], "full-size snapkv")
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
    # votes, pool and selection of every unit against the oracle
    G = wl.group

    def jobs():
        for b in range(B):
            qb = bf16_bits(x["q_win"][b])
            kb = bf16_bits(x["k"][b])
            for g in range(H):
                yield (b, g), (qb[g * G:(g + 1) * G], kb[g], n, wl.scale, wl.pool_kernel)

    checked = 0
    with oracle_pool.pool() as ex:
        for (b, g), pooled in oracle_pool.map_bounded(ex, oracle_pool.snapkv_unit, jobs()):
            check_selection(K[b, g, :wl.budget], pooled, wl.budget, f"snapkv b{b} g{g}")
            checked += 1
    assert checked == B * H
    announce(f"snapkv: {checked} units' selections match the oracle")

    # decode over the compacted cache: the 64 steps the workload runs, every
    # step of the first and the last request against the oracle
    Ld = se.dense_layout(H, C, D)
    MP = C // 16
    pt = (torch.arange(B, device=DEV)[:, None] * (H * MP) + torch.arange(MP, device=DEV)[None]).to(torch.int32)
    Pd = se.decode_params(B, wl.num_q_heads, MP, MP, wl.scale)
    wsd = workspace(se.se_sparse_decode_workspace_size(Ld, Pd))
    out = torch.empty((B, wl.num_q_heads, D), dtype=torch.float32, device=DEV)
    base = klen[:, 0].long()
    bi = torch.arange(B, device=DEV)
    results = []
    for s in range(wl.decode_steps):
        rows = base + s
        k_out[bi, :, rows] = x["k_steps"][s]
        v_out[bi, :, rows] = x["v_steps"][s]
        lens = (rows + 1).to(torch.int32)
        call_twice(lambda: se.se_sparse_decode(Ld, Pd, x["q_steps"][s], k_out, v_out, pt, None, lens, out, None,
                                               wsd), wsd, [out], f"snapkv step {s}")
        o = to_np(out)
        qs = bf16_bits(x["q_steps"][s])
        for b in (0, B - 1):
            n_b = int(lens[b])
            results.append(((s, b), (qs[b], bf16_bits(k_out[b, :, :n_b]), bf16_bits(v_out[b, :, :n_b]), n_b, G,
                                     wl.scale), o[b]))
    with oracle_pool.pool() as ex:
        want = dict(oracle_pool.map_bounded(ex, oracle_pool.decode_rows, ((k, a) for k, a, _ in results)))
    for (s, b), args, got in results:
        vmax = float(np.abs(oracle.bf16_to_f64(args[2][:, :args[3]])).max())
        check_attention(got, want[(s, b)], vmax, f"snapkv step {s} b{b}")


@pytest.mark.parametrize("name", ["h2o", "prune", "pyramid_layer0", "pyramid_layer3"])
def test_eviction_family_full_size_every_unit(name):
    """The H2O, prefix-pruning and PyramidKV legs at the size the bench runs
    (PyramidKV: its first and last layers' budgets): counts, forced tokens,
    bitwise copies, and votes and selection against the oracle, on every unit."""
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
    call_twice(lambda: se.se_snapkv_compact(p, x["q_win"], x["k"], x["v"], x["prompt_lens"], k_out, v_out, kept, klen,
                                            ws), ws, [k_out, v_out, kept, klen], f"full-size {wl.name}")
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
    G = wl.group

    def jobs():
        for b in range(B):
            qb = bf16_bits(x["q_win"][b])
            kb = bf16_bits(x["k"][b])
            for g in range(H):
                yield (b, g), (qb[g * G:(g + 1) * G], kb[g], n, wl.scale, wl.pool_kernel)

    checked = 0
    with oracle_pool.pool() as ex:
        for (b, g), pooled in oracle_pool.map_bounded(ex, oracle_pool.snapkv_unit, jobs()):
            check_selection(K[b, g, lo:lo + R] - lo, pooled[lo:hi], R, f"{wl.name} b{b} g{g}")
            checked += 1
    assert checked == B * H
    announce(f"{wl.name}: {checked} units' selections match the oracle")
