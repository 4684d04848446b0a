"""Quest decode over many steps with appends: each step writes the new
token's K/V into its request's last page (a new page every 16 tokens), counts
it in seq_lens and decodes with the fused last-page refresh.  The summaries
the library maintains this way must equal the oracle's, built from scratch on
the cache as it stands, bit for bit, at every step; the selection and the
attention are checked against the oracle at every step as well.  The second
case keeps every page (the dense policy a model applies to its first layers)
alternating with sparse steps on the same cache.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_long_amd as se
from synth import QuestWorkload, make_quest_inputs, bf16_bits
from gpu_util import (DEV, announce, build_summaries, check_attention, check_selection, host_inputs, layout_for,
                      run_sparse_decode, sel_lists, to_np)

pytestmark = pytest.mark.gpu

CASES = {
    "gqa_d128": (QuestWorkload("t_steps_gqa", 3, 16, 2, 128, 128, 160, 3, "none", seed=41), [30, 47, 16]),
    "mla": (QuestWorkload("t_steps_mla", 2, 32, 1, 576, 512, 128, 2, "none", v_is_k_prefix=True, seed=42), [15, 33]),
}


def _append(x, wl, step_rng):
    """Write one new token per request at position seq_lens[b] and count it."""
    lens = x["seq_lens"].clone()
    pt = x["page_table"]
    for b in range(wl.batch):
        n = int(lens[b])
        phys = int(pt[b, n // 16])
        krow = torch.from_numpy(step_rng.standard_normal((wl.num_kv_heads, wl.head_dim_qk))).float().to(DEV)
        x["k_pages"][phys, :, n % 16] = krow.to(torch.bfloat16)
        if x["v_pages"] is not None:
            vrow = torch.from_numpy(step_rng.standard_normal((wl.num_kv_heads, wl.head_dim_v))).float().to(DEV)
            x["v_pages"][phys, :, n % 16] = vrow.to(torch.bfloat16)
    x["seq_lens"] = (lens + 1).to(torch.int32)
    x["q"] = torch.from_numpy(step_rng.standard_normal((wl.batch, wl.num_q_heads, wl.head_dim_qk))).float().to(
        DEV).to(torch.bfloat16)


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_steps_with_appends_keep_summaries_exact(name):
    wl, lens0 = CASES[name]
    steps = 40
    announce(f"multistep {name} seed {wl.seed} lens {lens0} steps {steps}")
    x = make_quest_inputs(wl, DEV, poison_tail=True, seq_lens=lens0)
    summ = build_summaries(x, wl)
    rng = np.random.default_rng(wl.seed)
    vmax = 8.0
    for t in range(steps):
        _append(x, wl, rng)
        dense = name == "gqa_d128" and t % 4 == 3  # every fourth step keeps every page
        out, sel = run_sparse_decode(x, wl, summ, topk=wl.max_pages if dense else None, refresh=1)
        h = host_inputs(x)
        ref_summ = oracle.quest_summaries(h["k"], h["pt"], h["lens"])
        got = bf16_bits(summ).astype(np.uint16)
        for b, n in enumerate(h["lens"]):
            Pb = -(-int(n) // 16)
            for lp in range(Pb):
                phys = int(h["pt"][b, lp])
                for g in range(wl.num_kv_heads):
                    want = ref_summ[b, lp, g]  # fp64 [2, D], exact bf16 values
                    have = oracle.bf16_to_f64(got[phys, g])
                    assert (have == want).all(), f"{name} step {t} b{b} page {lp} g{g}: summary differs"
        A = oracle.quest_scores(h["q"], ref_summ, h["lens"], wl.group, wl.scale)
        sel_np = to_np(sel)
        k = wl.max_pages if dense else wl.topk
        for b, n in enumerate(h["lens"]):
            Pb = -(-int(n) // 16)
            for g in range(wl.num_kv_heads):
                check_selection(sel_np[b, g], A[b, g, :Pb], k, f"{name} step {t} b{b} g{g}")
        ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], sel_lists(sel_np, h["lens"]),
                                      wl.group, wl.scale, wl.head_dim_v, wl.v_is_k_prefix)
        check_attention(to_np(out), ref, vmax, f"{name} step {t}")
