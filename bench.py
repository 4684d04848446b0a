"""Throughput of the sparse-KV decode step on one MI355X.

Default workload: one attention layer's Quest decode step at 128K context
(batch 32, 32 query / 4 KV heads, head dim 128, 8192 16-token pages per
request, 256 pages kept per KV head), synthetic bf16 cache with Zipf key
saliency.  A step is the whole hot path: page scoring with the fused
last-page summary refresh, top-k per KV head, split-K attention over the kept
pages and the split merge.

Protocol: inputs are resident in HBM before timing; each timed step gets a
fresh query and is preceded (outside its events) by a 1 GiB read that evicts
the 256 MB Infinity Cache and the L2s with clean lines; step time comes from
HIP events on the launch stream.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "sparse decode tokens/s + effective HBM GB/s (% peak), 128K ctx, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa32x4_d128_128k_b32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=6, help="(request, KV head) units the oracle times")
    return ap.parse_args()


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_kv_long_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_record(kernel: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec or rec.get("sources_hash") != kernel_sources_hash():
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode path has no "
              f"multi-GPU form here: it would shard by request or KV head with no collective).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_kv_long_amd as se
    from synth import WORKLOADS, make_quest_inputs

    wl = WORKLOADS[args.workload]
    dev = "cuda"
    t0 = time.time()
    x = make_quest_inputs(wl, dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    B, Hq, Hkv, Dk, Dv, MP = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim_qk, wl.head_dim_v, wl.max_pages
    L = se.paged_layout(Hkv, Dk, Dv, wl.v_is_k_prefix)
    summ = torch.empty((x["k_pages"].shape[0], Hkv, 2, Dk), dtype=torch.bfloat16, device=dev)
    se.se_build_summaries(L, B, MP, x["k_pages"], x["page_table"], x["seq_lens"], summ)
    P = se.decode_params(B, Hq, MP, wl.topk, wl.scale, 0, 1, 0)
    ws = torch.empty(se.se_sparse_decode_workspace_size(L, P), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, Dv), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Hkv, wl.topk), dtype=torch.int32, device=dev)
    scores = torch.empty((B, Hkv, MP), dtype=torch.float32, device=dev)
    nq = 64
    gq = torch.Generator(device=dev)
    gq.manual_seed(wl.seed + 77)
    qs = torch.randn((nq, B, Hq, Dk), generator=gq, device=dev).to(torch.bfloat16)
    # cache flush: READ 1 GiB (4x the Infinity Cache) so the caches fill with
    # clean lines; a write flush would leave dirty lines whose write-back
    # then competes with the measured kernel
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    flush_sink = torch.empty((1,), dtype=torch.float32, device=dev)
    flush = None if args.no_flush else (lambda: torch.sum(flush_buf, dim=(0,), keepdim=True, out=flush_sink))
    torch.cuda.synchronize()

    lens = x["seq_lens"].cpu().numpy().astype(np.int64)
    pages = (lens + 15) // 16
    kept = np.minimum(pages, wl.topk)
    # algorithmic bytes of one step
    row_k = Dk * 2
    row_v = 0 if wl.v_is_k_prefix else Dv * 2
    tok_kept = sum(int(min(n, 16 * k)) if k == p else int(16 * k) for n, k, p in zip(lens, kept, pages))
    bytes_q = B * Hq * Dk * 2
    bytes_summ = int(pages.sum()) * Hkv * 2 * Dk * 2
    bytes_pt = int(pages.sum()) * 4
    bytes_kv = tok_kept * Hkv * (row_k + row_v)
    bytes_out = B * Hq * Dv * 4
    b_alg = bytes_q + bytes_summ + bytes_pt + bytes_kv + bytes_out
    bytes_k1 = bytes_q + bytes_summ + bytes_pt + int(pages.sum()) * Hkv * 4  # + scores written

    def step(i):
        q = qs[i % nq]
        se.se_sparse_decode(L, P, q, x["k_pages"], x["v_pages"], x["page_table"], summ, x["seq_lens"], out, sel, ws)

    def timed(fn, count, warm):
        for i in range(warm):
            if flush:
                flush()
            fn(i)
        torch.cuda.synchronize()
        evs = []
        wall0 = time.perf_counter()
        for i in range(count):
            if flush:
                flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn(i)
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms = np.array([a.elapsed_time(b) for a, b in evs])
        return ms, wall

    # whole step
    step_ms, wall = timed(step, args.steps, args.warmup)
    # per-step pieces, each timed alone on the same inputs
    def k1(i):
        se.se_quest_scores(L, P, qs[i % nq], x["k_pages"], x["page_table"], summ, x["seq_lens"], scores)

    def k2(i):
        se.se_topk_pages(P, Hkv, scores, x["seq_lens"], sel)

    def k34(i):
        se.se_decode_selected(L, P, qs[i % nq], x["k_pages"], x["v_pages"], x["page_table"], x["seq_lens"], sel, out,
                              ws)

    k1_ms, _ = timed(k1, args.steps, 2)
    k2_ms, _ = timed(k2, args.steps, 2)
    k34_ms, _ = timed(k34, args.steps, 2)

    t_step = float(np.mean(step_ms)) * 1e-3
    tokens_s = B / t_step
    gbps = b_alg / t_step / 1e9
    k1_s = float(np.mean(k1_ms)) * 1e-3
    k1_gbps = bytes_k1 / k1_s / 1e9
    t_k34 = float(np.mean(k34_ms)) * 1e-3
    bytes_k34 = bytes_q + bytes_kv + bytes_out
    k34_gbps = bytes_k34 / t_k34 / 1e9

    result = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "context": wl.context, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim_qk": Dk, "head_dim_v": Dv, "page_tokens": 16, "topk_pages": wl.topk,
                   "saliency": wl.saliency},
        "effective_hbm_gbps": round(gbps, 1),
        "pct_peak_hbm": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_step": b_alg,
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, p)), 4) for p in (10, 50, 90)],
        "wall_s_timed_loop_incl_flush": round(wall, 4),
        "cache_flush_between_steps": flush is not None,
        "pieces_ms": {"quest_scores": round(float(np.mean(k1_ms)), 4), "topk_pages": round(float(np.mean(k2_ms)), 4),
                      "decode_and_merge": round(float(np.mean(k34_ms)), 4)},
        "roofline": {"kernel": "quest_score (page scoring + last-page refresh)", "bound": "hbm",
                     "achieved": round(k1_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(k1_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic_record("quest_score"),
                     "algorithmic_bytes_per_launch": bytes_k1},
        "decode_kernel_gbps": round(k34_gbps, 1),
        "input_generation_s": round(gen_s, 1),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, x, summ, qs[0], args.cpu_units)
    print(json.dumps(result))


def cpu_baseline(wl, x, summ, q, units):
    """Time the oracle's decode step (page bounds, KV-head scores, selection,
    attention -- given the page summaries) on a few (request, KV head) units,
    single-threaded, and scale to the whole step."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from synth import bf16_bits

    G, D = wl.group, wl.head_dim_qk
    rng = np.random.default_rng(0)
    picks = [(int(b), int(g)) for b, g in zip(rng.integers(0, wl.batch, units), rng.integers(0, wl.num_kv_heads, units))]
    pt = x["page_table"].cpu().numpy()
    lens = x["seq_lens"].cpu().numpy()
    qh = bf16_bits(q)
    spent = 0.0
    for b, g in picks:
        n = int(lens[b])
        P = -(-n // 16)
        rows = torch_index(x["k_pages"], pt[b, :P], g)
        vrows = None if x["v_pages"] is None else torch_index(x["v_pages"], pt[b, :P], g)
        sm = bf16_bits(summ[pt[b, :P].astype(np.int64), g])  # [P, 2, D]
        mins, maxs = oracle.bf16_to_f64(sm[:, 0]), oracle.bf16_to_f64(sm[:, 1])
        kp = oracle.bf16_to_f64(rows)
        vp = kp[..., :wl.head_dim_v] if vrows is None else oracle.bf16_to_f64(vrows)
        qf = oracle.bf16_to_f64(qh[b, g * G:(g + 1) * G])
        with threadpool_limits(1):
            t0 = time.perf_counter()
            U = oracle.unit_page_bounds(qf, mins, maxs, wl.scale)
            A = oracle.unit_kv_head_score(U)
            s = oracle.unit_select(A, wl.topk)
            keys = oracle.unit_selected_tokens(kp, s, n)
            vals = oracle.unit_selected_tokens(vp, s, n)
            oracle.unit_attention(qf, keys, vals, wl.scale)
            spent += time.perf_counter() - t0
    per_unit = spent / len(picks)
    step_s = per_unit * wl.batch * wl.num_kv_heads
    return {"value": round(wl.batch / step_s, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(picks)} of {wl.batch * wl.num_kv_heads} (request, KV head) units of the same step, "
                      f"fp64 numpy single-threaded, page bounds + KV-head max + top-k + attention given the page "
                      f"summaries; {spent:.2f} s measured, scaled by units"}


def torch_index(pages, phys, g):
    import numpy as np
    import torch
    from synth import bf16_bits
    idx = torch.from_numpy(np.asarray(phys, dtype=np.int64)).to(pages.device)
    return bf16_bits(pages.index_select(0, idx)[:, g])


if __name__ == "__main__":
    main()
