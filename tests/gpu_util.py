"""Helpers shared by the GPU parity tests: run the library through its C ABI
and compare with the oracle under the stated tolerances.

Tolerances (floating point; selections and copies are compared exactly):
  * page scores: |gpu - oracle| <= 1e-5 * s * sum_c |q_c| * max(|min_c|, |max_c|)
    (fp32 accumulation of 2D exact bf16 products; the bound is the L1 size of
    the terms, so cancellation cannot defeat it).
  * selections: the gap rule -- with tau the oracle's k-th largest score and
    eps = 1e-3 * max(|tau|, 1e-12 * max|score|), every id scoring above
    tau + eps must be kept, none scoring below tau - eps may be, the count is
    exactly min(topk, pages) and ids are ascending and distinct.
  * attention outputs, against the oracle evaluated on the GPU's own
    selection: max abs error <= 2e-2 and mean abs error <= 2e-3, and the
    tighter fp32 bound max abs <= 2e-3 * max(1, max|v|).
  * SnapKV votes: relative error <= 2e-4 of each vote plus 1e-6 of the
    largest vote.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_kv_long_amd as se
from synth import bf16_bits

DEV = "cuda"

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def announce(msg: str):
    print(f"\n[gpu] {msg}", flush=True)


def layout_for(wl):
    return se.paged_layout(wl.num_kv_heads, wl.head_dim_qk, wl.head_dim_v, wl.v_is_k_prefix)


def to_np(t):
    return t.detach().to("cpu").numpy()


def build_summaries(x, wl):
    P = x["k_pages"].shape[0]
    summ = torch.full((P, wl.num_kv_heads, 2, wl.head_dim_qk), float("nan"), dtype=torch.bfloat16, device=DEV)
    se.se_build_summaries(layout_for(wl), wl.batch, wl.max_pages, x["k_pages"], x["page_table"], x["seq_lens"], summ)
    return summ


def params_for(wl, topk=None, refresh=1, splits=0, head_agg=0, sink=0, recent=0, valu=0):
    return se.decode_params(wl.batch, wl.num_q_heads, wl.max_pages, wl.topk if topk is None else topk, wl.scale,
                            head_agg, refresh, splits, sink, recent, valu)


# Workspace fills: 0xFF bytes read as fp32 NaN and int32 -1, zeros as 0.0 and
# 0.  Every call that takes a workspace runs once on each (call_twice), so a
# kernel that reads workspace memory its own call did not write sees two
# different values and the outputs differ.
FILL_FIRST, FILL_SECOND = 0xFF, 0x00


def workspace(nbytes):
    """A workspace buffer, filled with 0xFF bytes (NaN / -1)."""
    return torch.full((max(nbytes, 256),), FILL_FIRST, dtype=torch.uint8, device=DEV)


def call_twice(call, ws, outputs, what=""):
    """Run call() on a workspace filled with 0xFF bytes, then again on the same
    workspace filled with zeros; every tensor in `outputs` must come out
    bitwise identical (the second call recomputes them from the same inputs)."""
    ws.fill_(FILL_FIRST)
    call()
    torch.cuda.synchronize()
    first = [o.clone() for o in outputs]
    ws.fill_(FILL_SECOND)
    call()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(first, outputs)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
            f"{what}: output {i} depends on the workspace's prior contents"


def run_sparse_decode(x, wl, summ, topk=None, refresh=1, splits=0, head_agg=0, sink=0, recent=0, valu=0):
    P = params_for(wl, topk, refresh, splits, head_agg, sink, recent, valu)
    L = layout_for(wl)
    ws = workspace(se.se_sparse_decode_workspace_size(L, P))
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32, device=DEV)
    sel = torch.empty((wl.batch, wl.num_kv_heads, se.kept_capacity(P)), dtype=torch.int32, device=DEV)
    call_twice(lambda: se.se_sparse_decode(L, P, x["q"], x["k_pages"], x["v_pages"], x["page_table"], summ,
                                           x["seq_lens"], out, sel, ws), ws, [out, sel], "se_sparse_decode")
    return out, sel


def host_inputs(x):
    h = {
        "q": bf16_bits(x["q"]),
        "k": bf16_bits(x["k_pages"]),
        "v": None if x["v_pages"] is None else bf16_bits(x["v_pages"]),
        "pt": to_np(x["page_table"]),
        "lens": to_np(x["seq_lens"]),
    }
    return h


def score_tolerance(q_heads_f64, mins, maxs, scale):
    """Per-page tolerance of the KV-head score: 1e-5 of the largest L1 term size over the group."""
    mag = np.abs(q_heads_f64)[:, None, :] * np.maximum(np.abs(mins), np.abs(maxs))[None]
    return 1e-5 * scale * mag.sum(axis=2).max(axis=0) + 1e-30


def check_selection(sel_row, scores, topk, what=""):
    """Gap-rule check of one (request, KV head) selection against fp64 scores."""
    P = len(scores)
    k = min(topk, P)
    got = np.asarray(sel_row)
    ids = got[:k]
    assert (got[k:] == -1).all(), f"{what}: padding"
    assert ((ids >= 0) & (ids < P)).all(), f"{what}: ids out of range"
    assert (np.diff(ids) > 0).all(), f"{what}: not ascending/distinct"
    if k == P:
        assert (ids == np.arange(P)).all()
        return
    order = np.sort(scores)[::-1]
    tau = order[k - 1]
    eps = 1e-3 * max(abs(tau), 1e-12 * np.abs(scores).max())
    must = np.nonzero(scores > tau + eps)[0]
    kept = set(ids.tolist())
    assert set(must.tolist()) <= kept, f"{what}: missing ids above the gap"
    assert (scores[ids] >= tau - eps).all(), f"{what}: ids below the gap"


def check_forced_selection(sel_row, scores, topk, sink, recent, what=""):
    """A selection with always-kept pages: the first `sink` and last `recent`
    pages exactly, and among the other pages the gap rule for `topk`."""
    P = len(scores)
    cap = topk + sink + recent
    got = np.asarray(sel_row)
    forced = sorted({p for p in range(P) if p < sink or p >= P - recent})
    others = np.array([p for p in range(P) if p not in set(forced)], dtype=np.int64)
    k = min(cap, P)
    ids = got[:k]
    assert len(got) == cap and (got[k:] == -1).all(), f"{what}: padding"
    assert (np.diff(ids) > 0).all() and ((ids >= 0) & (ids < P)).all(), f"{what}: not ascending ids in range"
    assert set(forced) <= set(ids.tolist()), f"{what}: a forced page is missing"
    picked = np.array(sorted(set(ids.tolist()) - set(forced)), dtype=np.int64)
    assert len(picked) == min(topk, len(others)), f"{what}: wrong number of selected pages"
    if len(picked) == 0 or len(picked) == len(others):
        return
    # gap rule among the non-forced pages, in their own index space
    pos = {int(p): i for i, p in enumerate(others)}
    row = np.full(topk, -1, dtype=np.int64)
    row[:len(picked)] = [pos[int(p)] for p in picked]
    check_selection(row, scores[others], topk, what)


def check_attention(out_gpu, out_ref, vmax, what=""):
    err = np.abs(np.asarray(out_gpu, np.float64) - out_ref)
    assert np.isfinite(out_gpu).all(), f"{what}: non-finite output"
    assert err.max() <= 2e-2, f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= 2e-3, f"{what}: mean abs err {err.mean():.3e}"
    assert err.max() <= 2e-3 * max(1.0, vmax), f"{what}: max abs err {err.max():.3e} > fp32 bound"
    return float(err.max()), float(err.mean())


def sel_lists(sel_np, lens, page=16):
    """GPU selection [B, Hkv, topk] -> nested lists without the -1 padding."""
    B, Hkv, _ = sel_np.shape
    out = []
    for b in range(B):
        out.append([sel_np[b, g][sel_np[b, g] >= 0] for g in range(Hkv)])
    return out
