"""The decode path under HIP graph capture: a captured se_sparse_decode,
replayed several times with fresh queries and eager GPU work in between, must
reproduce the eager call bit for bit on every replay."""
import pytest
import torch

import sparse_kv_long_amd as se
from synth import QuestWorkload, make_quest_inputs
from gpu_util import DEV, announce, build_summaries, layout_for, params_for, workspace

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("topk", [12, 1000])  # sparse, and dense over every page
def test_captured_decode_replays_match_eager(topk):
    wl = QuestWorkload("t_graph", 3, 16, 2, 128, 128, 1500, topk, "zipf", seed=41)
    announce(f"graph capture topk {topk}")
    x = make_quest_inputs(wl, DEV, seq_lens=[1500, 777, 33])
    summ = build_summaries(x, wl)
    L = layout_for(wl)
    P = params_for(wl, refresh=0)
    ws = workspace(se.se_sparse_decode_workspace_size(L, P))
    q = x["q"].clone()
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32, device=DEV)

    def call():
        se.se_sparse_decode(L, P, q, x["k_pages"], x["v_pages"], x["page_table"], summ, x["seq_lens"], out, None, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    for rep in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(torch.bfloat16))
        call()  # eager
        torch.cuda.synchronize()
        want = out.clone()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep} differs from the eager call"
