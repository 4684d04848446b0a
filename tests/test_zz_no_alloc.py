"""se_sparse_decode_noalloc: the decode step with its workspace in the
library's own device array, for callers that cannot allocate.  Two calls in
a row, the second on a smaller input and another stream, each bitwise equal
to se_sparse_decode on the same inputs (the same kernels, so the same bits)
and within the attention tolerance of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_kv_long_amd as se
from synth import QuestWorkload, make_quest_inputs
from gpu_util import (DEV, announce, build_summaries, check_attention, check_selection, host_inputs, layout_for,
                      params_for, run_sparse_decode, sel_lists, to_np)

pytestmark = pytest.mark.gpu

CALLS = [
    # (workload, lengths, stream): a GQA batch, then a smaller latent-attention one
    (QuestWorkload("t_noalloc_gqa", 3, 16, 2, 128, 128, 1500, 20, "zipf", seed=61), [1500, 1, 229], False),
    (QuestWorkload("t_noalloc_mla", 1, 32, 1, 576, 512, 600, 6, "none", v_is_k_prefix=True, seed=62), [583], True),
]


def test_noalloc_matches_workspace_entry_point_twice():
    for i, (wl, lens, side) in enumerate(CALLS):
        announce(f"no-alloc call {i}: {wl.name} lens {lens} side stream {side}")
        x = make_quest_inputs(wl, DEV, poison_tail=True, seq_lens=lens)
        summ = build_summaries(x, wl)
        want_out, want_sel = run_sparse_decode(x, wl, summ)
        L, P = layout_for(wl), params_for(wl)
        assert se.se_sparse_decode_workspace_size(L, P) <= se.NOALLOC_SCRATCH_BYTES
        out = torch.full_like(want_out, float("nan"))
        sel = torch.full_like(want_sel, 12345)
        stream = torch.cuda.Stream() if side else torch.cuda.current_stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            se.se_sparse_decode_noalloc(L, P, x["q"], x["k_pages"], x["v_pages"], x["page_table"], summ,
                                        x["seq_lens"], out, sel)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want_out.view(torch.int32)), f"call {i}: output"
        assert torch.equal(sel, want_sel), f"call {i}: selection"
        h = host_inputs(x)
        ref_summ = oracle.quest_summaries(h["k"], h["pt"], h["lens"])
        A = oracle.quest_scores(h["q"], ref_summ, h["lens"], wl.group, wl.scale)
        sel_np = to_np(sel)
        for b, n in enumerate(h["lens"]):
            for g in range(wl.num_kv_heads):
                check_selection(sel_np[b, g], A[b, g, :-(-int(n) // 16)], wl.topk, f"no-alloc {i} b{b} g{g}")
        ref = oracle.sparse_attention(h["q"], h["k"], h["v"], h["pt"], h["lens"], sel_lists(sel_np, h["lens"]),
                                      wl.group, wl.scale, wl.head_dim_v, wl.v_is_k_prefix)
        vmax = float(torch.nan_to_num(x["v_pages"] if x["v_pages"] is not None else x["k_pages"], 0.0).abs().max())
        check_attention(to_np(out), ref, vmax, f"no-alloc call {i}")


def test_noalloc_rejects_a_step_beyond_the_array():
    """A step whose workspace exceeds the array is refused before any launch."""
    L = se.paged_layout(4, 128, 128)
    P = se.decode_params(32, 32, 65536, 256)
    assert se.se_sparse_decode_workspace_size(L, P) > se.NOALLOC_SCRATCH_BYTES
    t = torch.empty(64, dtype=torch.uint8, device=DEV)
    p = t.data_ptr()
    rc = se.lib().se_sparse_decode_noalloc(ctypes.byref(L), ctypes.byref(P), p, p, p, p, p, p, p, None,
                                           torch.cuda.current_stream().cuda_stream)
    assert rc == se.SE_EWORKSPACE


def test_noalloc_under_graph_capture():
    """The callers the entry point is for: a captured se_sparse_decode_noalloc,
    replayed with fresh queries and eager work in between, reproduces the
    eager call bit for bit on every replay."""
    wl = QuestWorkload("t_noalloc_graph", 3, 16, 2, 128, 128, 1500, 12, "zipf", seed=63)
    announce("no-alloc graph capture")
    x = make_quest_inputs(wl, DEV, seq_lens=[1500, 777, 33])
    summ = build_summaries(x, wl)
    L, P = layout_for(wl), params_for(wl, refresh=0)
    q = x["q"].clone()
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32, device=DEV)
    sel = torch.empty((wl.batch, wl.num_kv_heads, wl.topk), dtype=torch.int32, device=DEV)

    def call():
        se.se_sparse_decode_noalloc(L, P, q, x["k_pages"], x["v_pages"], x["page_table"], summ, x["seq_lens"], out,
                                    sel)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # the first call on this GPU looks up the array's address, outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(9)
    for rep in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(torch.bfloat16))
        call()  # eager
        torch.cuda.synchronize()
        want_out, want_sel = out.clone(), sel.clone()
        out.fill_(float("nan"))
        sel.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_out), f"replay {rep}: output differs from the eager call"
        assert torch.equal(sel, want_sel), f"replay {rep}: selection differs from the eager call"
