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
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time each oracle-baseline worker spends on its sampled (request, KV head) units")
    ap.add_argument("--topk", type=int, default=None, help="pages selected by score (default: the workload's)")
    ap.add_argument("--sink-pages", type=int, default=0, help="leading pages every request always keeps")
    ap.add_argument("--recent-pages", type=int, default=0, help="trailing pages every request always keeps")
    ap.add_argument("--valu-attention", action="store_true",
                    help="run the attention on the vector-ALU kernel instead of the matrix cores")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (HBM byte-counter calibration)")
    return ap.parse_args()


# Source files each recorded kernel is built from (beside the shared headers
# and the build flags): a counter record stays valid while these are unchanged.
KERNEL_SOURCES = {"quest_score": ["quest.hip"], "topk_pages": ["topk.hip"], "decode": ["decode.hip"],
                  "merge": ["decode.hip"], "snapkv_votes": ["snapkv.hip"]}


def kernel_sources_hash(kernel: str) -> str:
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "sparse_kv_long_amd")
    files = [os.path.join("csrc", f) for f in KERNEL_SOURCES[kernel] + ["common.h", "se_internal.h"]] + ["build.py"]
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(pkg, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_record(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken for this workload on the kernel's current sources (else None)."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}@{workload}")
    if not rec or rec.get("sources_hash") != kernel_sources_hash(kernel):
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

    if args.copy_calibration:
        copy_calibration(torch)
        return

    import sparse_kv_long_amd as se
    from synth import WORKLOADS, SnapKVWorkload, make_quest_inputs

    wl = WORKLOADS[args.workload]
    if isinstance(wl, SnapKVWorkload) and wl.layers > 1:
        bench_pyramid(args, wl)
        return
    if isinstance(wl, SnapKVWorkload):
        bench_snapkv(args, wl)
        return
    dev = "cuda"
    t0 = time.time()
    x = make_quest_inputs(wl, dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    B, Hq, Hkv, Dk, Dv, MP = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim_qk, wl.head_dim_v, wl.max_pages
    L = se.paged_layout(Hkv, Dk, Dv, wl.v_is_k_prefix)
    summ = torch.empty((x["k_pages"].shape[0], Hkv, 2, Dk), dtype=torch.bfloat16, device=dev)
    se.se_build_summaries(L, B, MP, x["k_pages"], x["page_table"], x["seq_lens"], summ)
    topk = wl.topk if args.topk is None else args.topk
    sink, recent = args.sink_pages, args.recent_pages
    forced = sink > 0 or recent > 0 or topk != wl.topk or args.valu_attention
    # topk = 0 keeps the forced pages only: nothing is scored or refreshed
    P = se.decode_params(B, Hq, MP, topk, wl.scale, 0, 1 if topk > 0 else 0, 0, sink, recent,
                         valu_attention=int(args.valu_attention))
    kcap = se.kept_capacity(P)
    ws = torch.empty(se.se_sparse_decode_workspace_size(L, P), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, Dv), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Hkv, kcap), dtype=torch.int32, device=dev)
    scores = torch.empty((B, Hkv, MP), dtype=torch.float32, device=dev)
    nq = 64
    gq = torch.Generator(device=dev)
    gq.manual_seed(wl.seed + 77)
    qs = torch.randn((nq, B, Hq, Dk), generator=gq, device=dev).to(torch.bfloat16)
    # cache flush: READ 1 GiB (4x the Infinity Cache) so the caches fill with
    # clean lines; a write flush would leave dirty lines whose write-back
    # then competes with the measured kernel
    flush = make_flush(torch, not args.no_flush)
    torch.cuda.synchronize()

    lens = x["seq_lens"].cpu().numpy().astype(np.int64)
    scored = topk > 0
    alg = quest_algorithmic_bytes(lens, Hq, Hkv, Dk, Dv, wl.v_is_k_prefix, topk, kcap, recent)
    b_alg, bytes_k1 = alg["step"], alg["scorer_launch"]
    bytes_q, bytes_kv, bytes_out = alg["q"], alg["kv"], alg["out"]

    def step(i):
        q = qs[i % nq]
        se.se_sparse_decode(L, P, q, x["k_pages"], x["v_pages"], x["page_table"], summ if scored else None,
                            x["seq_lens"], out, sel, ws)

    def timed(fn, count, warm):
        return timed_calls(fn, count, warm, flush)

    # whole step
    step_ms, wall = timed(step, args.steps, args.warmup)
    # the same step with warm caches (no flush), for information
    hot_ms, _ = timed_calls(step, args.steps, 2, None)
    # per-step pieces, each timed alone on the same inputs
    def k1(i):
        se.se_quest_scores(L, P, qs[i % nq], x["k_pages"], x["page_table"], summ, x["seq_lens"], scores)

    def k2(i):
        se.se_topk_pages(P, Hkv, scores, x["seq_lens"], sel)

    def k34(i):
        se.se_decode_selected(L, P, qs[i % nq], x["k_pages"], x["v_pages"], x["page_table"], x["seq_lens"], sel, out,
                              ws)

    k1_ms, _ = timed(k1, args.steps, 2) if scored else (np.zeros(1), 0.0)
    k2_ms, _ = timed(k2, args.steps, 2)
    k34_ms, _ = timed(k34, args.steps, 2)

    t_step = float(np.mean(step_ms)) * 1e-3
    tokens_s = B / t_step
    gbps = b_alg / t_step / 1e9
    k1_s = float(np.mean(k1_ms)) * 1e-3
    k1_gbps = bytes_k1 / k1_s / 1e9 if scored else 0.0
    t_k34 = float(np.mean(k34_ms)) * 1e-3
    bytes_k34 = bytes_q + bytes_kv + bytes_out
    k34_gbps = bytes_k34 / t_k34 / 1e9

    variant = f", sink {sink} + recent {recent} + top {topk} pages" if (sink or recent or topk != wl.topk) else ""
    if args.valu_attention:
        variant += ", vector-ALU attention"
    if scored:
        roofline = {"kernel": "quest_score (page scoring + last-page refresh)", "bound": "hbm",
                    "achieved": round(k1_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(k1_gbps / HBM_PEAK_GBPS, 4),
                    # the stored counters were taken on the workload's own selection budget
                    "traffic": None if forced else traffic_record("quest_score", wl.name),
                    "algorithmic_bytes_per_launch": bytes_k1}
    else:  # nothing scored: the decode is the dominant kernel
        roofline = {"kernel": "decode over the kept pages + split merge", "bound": "hbm",
                    "achieved": round(k34_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(k34_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                    "algorithmic_bytes_per_launch": bytes_k34}
    result = {
        "metric": (METRIC if wl.name == "gqa32x4_d128_128k_b32" and not forced else
                   f"sparse decode tokens/s + effective HBM GB/s (% peak), {wl.name}{variant}, 1 GPU"),
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
                   "head_dim_qk": Dk, "head_dim_v": Dv, "page_tokens": 16, "topk_pages": topk,
                   "sink_pages": sink, "recent_pages": recent, "saliency": wl.saliency,
                   "attention_kernel": "vector ALU" if args.valu_attention else "matrix cores where built"},
        "effective_hbm_gbps": round(gbps, 1),
        "pct_peak_hbm": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_step": b_alg,
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, p)), 4) for p in (10, 50, 90)],
        "step_ms_hot_p50": round(float(np.median(hot_ms)), 4),
        "wall_s_timed_loop_incl_flush": round(wall, 4),
        "cache_flush_between_steps": flush is not None,
        **stream_read_reference(torch, gbps),
        "pieces_ms": {"quest_scores": round(float(np.mean(k1_ms)), 4), "topk_pages": round(float(np.mean(k2_ms)), 4),
                      "decode_and_merge": round(float(np.mean(k34_ms)), 4)},
        "roofline": roofline,
        "decode_kernel_gbps": round(k34_gbps, 1),
        # the bytes the step's kernels actually move (rocprofv3 FETCH_SIZE +
        # WRITE_SIZE per launch, calibrated), over the measured step time
        **counted_bytes(wl.name, t_step, forced),
        "input_generation_s": round(gen_s, 1),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, x, qs, args.cpu_seconds, topk, sink, recent)
    print(json.dumps(result))


def quest_algorithmic_bytes(lens, Hq, Hkv, Dk, Dv, v_is_k_prefix, topk, kcap, recent=0) -> dict:
    """The bytes one Quest decode step must move (q, the summaries of every
    valid page, the page table, the valid tokens of the kept pages' K and V
    -- the latent row once when V is a prefix of K -- and the output), and
    those of one scorer launch (q, summaries, page table).
    A kept partial last page counts its valid tokens when it is kept for
    sure (all pages kept, or recent pages forced), else 16 tokens."""
    lens = [int(n) for n in lens]
    B = len(lens)
    pages = [(n + 15) // 16 for n in lens]
    kept = [min(p, kcap) for p in pages]
    row = Dk * 2 + (0 if v_is_k_prefix else Dv * 2)
    tok_kept = sum(16 * (k - 1) + n - 16 * (p - 1) if (k == p or recent > 0) else 16 * k
                   for n, k, p in zip(lens, kept, pages))
    scored = topk > 0
    q = B * Hq * Dk * 2
    summ = sum(pages) * Hkv * 2 * Dk * 2 if scored else 0
    pt = sum(pages) * 4 if scored else sum(kept) * 4
    kv = tok_kept * Hkv * row
    out = B * Hq * Dv * 4
    # one scorer launch reads q, the summaries and the page table; the page
    # scores it writes are an intermediate of the step and are not counted
    return {"q": q, "summaries": summ, "page_table": pt, "kv": kv, "out": out, "step": q + summ + pt + kv + out,
            "scorer_launch": q + summ + pt}


def counted_bytes(workload: str, t_step: float, forced: bool) -> dict:
    recs = [traffic_record(k, workload) for k in ("quest_score", "topk_pages", "decode", "merge")]
    if forced or any(r is None for r in recs):
        return {"counted_hbm_bytes_per_step": None, "counted_hbm_gbps": None, "pct_peak_hbm_counted": None}
    total = int(sum(recs))
    gbps = total / t_step / 1e9
    return {"counted_hbm_bytes_per_step": total, "counted_hbm_gbps": round(gbps, 1),
            "pct_peak_hbm_counted": round(100 * gbps / HBM_PEAK_GBPS, 2)}


def timed_calls(fn, count, warm, flush):
    """Run fn(i) `warm` times, then `count` times each bracketed by HIP events
    on the current stream (the one the library launches on); `flush` (if
    any) runs before every call, outside the events."""
    import numpy as np
    import torch
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


def stream_read_reference(torch, gbps):
    """The rate of a plain streaming read on this GPU (`se_hbm_read` from
    libse_hbmread.so: 1 GiB read once, 16 B per lane per load; the best of a
    few grid sizes, median of 10 event-timed calls each) and the step's
    effective rate as a fraction of it."""
    import ctypes
    import numpy as np
    from stream_read.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: build it first (python -m stream_read.build)")
    h = ctypes.CDLL(PROBE_LIB)
    h.se_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    h.se_hbm_read.restype = ctypes.c_int
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros((1,), dtype=torch.int32, device="cuda")
    best, best_blocks = 0.0, 0
    for blocks in (1024, 4096, 16384, 65536):
        def read(i):
            rc = h.se_hbm_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"se_hbm_read failed: {rc}")
        ms, _ = timed_calls(read, 10, 3, None)
        rate = nbytes / (float(np.median(ms)) * 1e-3) / 1e9
        if rate > best:
            best, best_blocks = rate, blocks
    del buf
    return {"stream_read_gbps": round(best, 1), "frac_of_stream_read": round(gbps / best, 4),
            "stream_read_kernel": f"se_hbm_read, 1 GiB, {best_blocks} blocks of 256 threads"}


def make_flush(torch, enabled):
    """A 1 GiB read (4x the Infinity Cache): evicts the caches with clean lines
    (a write flush would leave dirty lines whose write-back then competes
    with the measured kernel)."""
    if not enabled:
        return None
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_sink = torch.empty((1,), dtype=torch.float32, device="cuda")
    return lambda: torch.sum(flush_buf, dim=(0,), keepdim=True, out=flush_sink)


def bench_snapkv(args, wl):
    """SnapKV eviction of a 32K-token prompt (window votes, pool, select,
    compaction) followed by the decode steps over the compacted cache.  One
    step = one eviction + all decode steps for the batch; tokens/s counts the
    decode tokens produced.  The caches are flushed before the eviction only:
    the compacted cache is small enough to stay in the Infinity Cache between
    decode steps, as it would in serving."""
    import numpy as np
    import torch

    import sparse_kv_long_amd as se
    from synth import make_snapkv_inputs

    dev = "cuda"
    t0 = time.time()
    x = make_snapkv_inputs(wl, dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    B, Hq, H, D, W, R = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window, wl.budget
    n = wl.prompt
    S = wl.decode_steps
    p = se.snapkv_params(B, Hq, H, D, n, W, wl.pool_kernel, R, 1 << 30, wl.scale, sink=wl.sink, recent=wl.recent,
                         interval=wl.interval)
    kcap = se.se_snapkv_kept_capacity(p)
    C = (kcap + S + 15) // 16 * 16  # kept rows plus the decode steps, whole pages
    p.out_capacity = C
    ws = torch.empty(se.se_snapkv_workspace_size(p), dtype=torch.uint8, device=dev)
    k_out = torch.zeros((B, H, C, D), dtype=torch.bfloat16, device=dev)
    v_out = torch.zeros((B, H, C, D), dtype=torch.bfloat16, device=dev)
    kept = torch.empty((B, H, kcap), dtype=torch.int32, device=dev)
    klen = torch.empty((B, H), dtype=torch.int32, device=dev)
    se.se_snapkv_compact(p, x["q_win"], x["k"], x["v"], x["prompt_lens"], k_out, v_out, kept, klen, ws)
    torch.cuda.synchronize()
    kl = int(klen[0, 0])
    assert (klen == kl).all() and kl <= kcap
    # the decode steps' tokens go in at rows kl..kl+steps-1 (the engine's
    # append); the eviction writes only rows < kept_len, so they are placed
    # once, outside the timing
    k_out[:, :, kl:kl + S] = x["k_steps"].permute(1, 2, 0, 3)
    v_out[:, :, kl:kl + S] = x["v_steps"].permute(1, 2, 0, 3)
    MP = C // 16
    pt = (torch.arange(B, device=dev)[:, None] * (H * MP) + torch.arange(MP, device=dev)[None]).to(torch.int32)
    Ld = se.dense_layout(H, C, D)
    Pd = se.decode_params(B, Hq, MP, MP, wl.scale)
    wsd = torch.empty(se.se_sparse_decode_workspace_size(Ld, Pd), dtype=torch.uint8, device=dev)
    out = torch.empty((S, B, Hq, D), dtype=torch.float32, device=dev)
    lens = [torch.full((B,), kl + s + 1, dtype=torch.int32, device=dev) for s in range(S)]
    flush = make_flush(torch, not args.no_flush)
    torch.cuda.synchronize()

    def evict(i):
        se.se_snapkv_compact(p, x["q_win"], x["k"], x["v"], x["prompt_lens"], k_out, v_out, kept, klen, ws)

    def decode_all(i):
        for s in range(S):
            se.se_sparse_decode(Ld, Pd, x["q_steps"][s], k_out, v_out, pt, None, lens[s], out[s], None, wsd)

    # the decode steps run as one captured HIP graph: 64 short steps issued
    # one by one from Python would time the host, not the GPU (the calls
    # allocate nothing and never synchronise, so they capture as they are)
    eager = out.clone()
    decode_all(0)
    torch.cuda.synchronize()
    eager.copy_(out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode_all(0)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_all(0)
    out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager), "graph replay differs from the eager decode steps"

    def decode_graph(i):
        graph.replay()

    def whole(i):
        evict(i)
        decode_graph(i)

    steps = max(1, args.steps // 5)
    whole_ms, wall = timed_calls(whole, steps, 2, flush)
    ev_ms, _ = timed_calls(evict, steps, 1, flush)
    votes = torch.empty((B, H, n), dtype=torch.float32, device=dev)
    vo_ms, _ = timed_calls(lambda i: se.se_snapkv_votes(p, x["q_win"], x["k"], x["prompt_lens"], votes, ws), steps, 1,
                           flush)
    dec_ms, _ = timed_calls(decode_graph, steps, 1, None)

    # re-eviction after the decode steps (the pages evict again every 1,024
    # decode steps): the same budget over the kept rows plus the steps, the
    # last W decode queries as the window, original positions carried through
    n2 = kl + S
    p2 = se.snapkv_params(B, Hq, H, D, C, W, wl.pool_kernel, R, 1 << 30, wl.scale, sink=wl.sink,
                          recent=wl.recent)
    kcap2 = se.se_snapkv_kept_capacity(p2)
    p2.out_capacity = (kcap2 + 15) // 16 * 16
    ws2 = torch.empty(se.se_snapkv_workspace_size(p2), dtype=torch.uint8, device=dev)
    k2 = torch.zeros((B, H, p2.out_capacity, D), dtype=torch.bfloat16, device=dev)
    v2 = torch.zeros_like(k2)
    kept2 = torch.empty((B, H, kcap2), dtype=torch.int32, device=dev)
    klen2 = torch.empty((B, H), dtype=torch.int32, device=dev)
    positions = torch.full((B, H, C), -1, dtype=torch.int32, device=dev)
    positions[:, :, :kl] = kept[:, :, :kl]
    positions[:, :, kl:n2] = torch.arange(n, n + S, dtype=torch.int32, device=dev)
    q_win2 = x["q_steps"][S - W:].permute(1, 2, 0, 3).contiguous() if S >= W else None
    lens2 = torch.full((B,), n2, dtype=torch.int32, device=dev)
    re_ms = None
    if q_win2 is not None:
        re_ms, _ = timed_calls(lambda i: se.se_snapkv_recompact(p2, q_win2, k_out, v_out, lens2, positions, k2, v2,
                                                                kept2, klen2, ws2), steps, 1, flush)

    t_whole = float(np.mean(whole_ms)) * 1e-3
    tokens_s = B * S / t_whole
    # algorithmic bytes: the window queries, K once, the kept K/V rows read and
    # written, the kept ids; then per decode step the attended rows, q and out
    b_evict, b_dec, b_votes = snapkv_algorithmic_bytes(B, Hq, H, D, n, W, kl, S)
    # window x context scores: pass 1 over every key, pass 2 over the columns
    # whose votes the selection reads (the candidates plus the pooling halo)
    ib, ie = wl.interval if wl.interval[1] else (0, n)
    lo, hi = max(wl.sink, ib), min(n - max(wl.recent, W), ie)
    vcols = min(hi + wl.pool_kernel // 2, n - W) - max(lo - wl.pool_kernel // 2, 0)
    flops_votes = 2 * B * Hq * W * D * (n + (n - W))  # se_snapkv_votes scores every prefix column
    t_votes = float(np.mean(vo_ms)) * 1e-3
    t_ev = float(np.mean(ev_ms)) * 1e-3
    t_dec = float(np.mean(dec_ms)) * 1e-3
    result = {
        "metric": f"{wl.method} eviction + decode tokens/s over the compacted cache, 32K prompt, 1 GPU",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": 2,
        "ms_per_step": round(t_whole * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "method": wl.method, "batch": B, "prompt": n, "num_q_heads": Hq,
                   "num_kv_heads": H, "head_dim": D, "window": W, "pool_kernel": wl.pool_kernel, "budget": R,
                   "sink": wl.sink, "recent": wl.recent, "interval": list(wl.interval), "kept_tokens": kl,
                   "decode_steps": S},
        "effective_hbm_gbps": round((b_evict + b_dec) / t_whole / 1e9, 1),
        "algorithmic_bytes_per_step": b_evict + b_dec,
        "pieces_ms": {"eviction": round(t_ev * 1e3, 4), "votes_only": round(t_votes * 1e3, 4),
                      "decode_steps_total": round(t_dec * 1e3, 4), "decode_step_mean": round(t_dec * 1e3 / S, 5),
                      "reeviction_after_steps": None if re_ms is None else round(float(np.mean(re_ms)), 4)},
        "eviction_vote_columns_pass2": vcols,
        "eviction_gbps": round(b_evict / t_ev / 1e9, 1),
        "decode_gbps_cache_resident": round(b_dec / t_dec / 1e9, 1),
        "roofline": votes_roofline(b_votes, flops_votes, t_votes, traffic_record("snapkv_votes", wl.name)),
        "cache_flush_before_eviction": flush is not None,
        "decode_steps_as_hip_graph": True,
        "wall_s_timed_loop_incl_flush": round(wall, 4),
        "input_generation_s": round(gen_s, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_snapkv(wl, x, args.cpu_seconds)
    print(json.dumps(result))


def bench_pyramid(args, wl):
    """PyramidKV over a slice of `wl.layers` layers: each layer evicts the
    32K prompt with its own budget from se_pyramid_budgets (the same sink,
    recent and window in every layer), then the decode steps run through
    every layer's retained cache.  One step = every layer's eviction + every
    layer's decode steps; tokens/s counts the decode tokens produced (each
    passes through all the layers).  The layers share one synthetic cache."""
    import numpy as np
    import torch

    import sparse_kv_long_amd as se
    from synth import make_snapkv_inputs

    dev = "cuda"
    t0 = time.time()
    x = make_snapkv_inputs(wl, dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    B, Hq, H, D, W, n, S = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window, wl.prompt, wl.decode_steps
    budgets = se.se_pyramid_budgets(wl.layers, wl.budget, *wl.layer_ratios)
    layers = []
    for R in budgets:
        p = se.snapkv_params(B, Hq, H, D, n, W, wl.pool_kernel, max(R, 1), 1 << 30, wl.scale, sink=wl.sink,
                             recent=wl.recent)
        kcap = se.se_snapkv_kept_capacity(p)
        C = (kcap + S + 15) // 16 * 16
        p.out_capacity = C
        st = {"p": p, "R": R, "C": C,
              "ws": torch.empty(se.se_snapkv_workspace_size(p), dtype=torch.uint8, device=dev),
              "k_out": torch.zeros((B, H, C, D), dtype=torch.bfloat16, device=dev),
              "v_out": torch.zeros((B, H, C, D), dtype=torch.bfloat16, device=dev),
              "kept": torch.empty((B, H, kcap), dtype=torch.int32, device=dev),
              "klen": torch.empty((B, H), dtype=torch.int32, device=dev)}
        se.se_snapkv_compact(p, x["q_win"], x["k"], x["v"], x["prompt_lens"], st["k_out"], st["v_out"], st["kept"],
                             st["klen"], st["ws"])
        torch.cuda.synchronize()
        kl = int(st["klen"][0, 0])
        assert (st["klen"] == kl).all()
        st["kl"] = kl
        st["k_out"][:, :, kl:kl + S] = x["k_steps"].permute(1, 2, 0, 3)
        st["v_out"][:, :, kl:kl + S] = x["v_steps"].permute(1, 2, 0, 3)
        MP = C // 16
        st["pt"] = (torch.arange(B, device=dev)[:, None] * (H * MP) + torch.arange(MP, device=dev)[None]).to(torch.int32)
        st["Ld"] = se.dense_layout(H, C, D)
        st["Pd"] = se.decode_params(B, Hq, MP, MP, wl.scale)
        st["wsd"] = torch.empty(se.se_sparse_decode_workspace_size(st["Ld"], st["Pd"]), dtype=torch.uint8, device=dev)
        st["lens"] = [torch.full((B,), kl + s + 1, dtype=torch.int32, device=dev) for s in range(S)]
        layers.append(st)
    out = torch.empty((S, B, Hq, D), dtype=torch.float32, device=dev)
    flush = make_flush(torch, not args.no_flush)

    def evict_all(i):
        for st in layers:
            se.se_snapkv_compact(st["p"], x["q_win"], x["k"], x["v"], x["prompt_lens"], st["k_out"], st["v_out"],
                                 st["kept"], st["klen"], st["ws"])

    def decode_all(i):
        # step s runs through every layer before step s + 1 (the model's order)
        for s in range(S):
            for st in layers:
                se.se_sparse_decode(st["Ld"], st["Pd"], x["q_steps"][s], st["k_out"], st["v_out"], st["pt"], None,
                                    st["lens"][s], out[s], None, st["wsd"])

    decode_all(0)
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode_all(0)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_all(0)
    out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager), "graph replay differs from the eager decode steps"

    def whole(i):
        evict_all(i)
        graph.replay()

    steps = max(1, args.steps // 10)
    whole_ms, wall = timed_calls(whole, steps, 1, flush)
    ev_ms, _ = timed_calls(evict_all, steps, 1, flush)
    dec_ms, _ = timed_calls(lambda i: graph.replay(), steps, 1, None)
    t_whole = float(np.mean(whole_ms)) * 1e-3
    t_ev = float(np.mean(ev_ms)) * 1e-3
    t_dec = float(np.mean(dec_ms)) * 1e-3
    kls = [st["kl"] for st in layers]
    b_evict = sum(B * Hq * W * D * 2 + B * H * n * D * 2 + 2 * 2 * B * H * kl * D * 2 + B * H * kl * 4 for kl in kls)
    b_dec = sum(B * H * sum(kl + s + 1 for s in range(S)) * 2 * D * 2 + S * (B * Hq * D * 2 + B * Hq * D * 4)
                for kl in kls)
    result = {
        "metric": f"PyramidKV eviction + decode tokens/s through a {wl.layers}-layer slice, 32K prompt, 1 GPU",
        "value": round(B * S / t_whole, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": 1,
        "ms_per_step": round(t_whole * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "method": wl.method, "layers": wl.layers,
                   "layer_ratios": list(wl.layer_ratios), "layer_budgets": budgets, "kept_tokens": kls,
                   "batch": B, "prompt": n, "num_q_heads": Hq, "num_kv_heads": H, "head_dim": D, "window": W,
                   "pool_kernel": wl.pool_kernel, "sink": wl.sink, "recent": wl.recent, "decode_steps": S},
        "effective_hbm_gbps": round((b_evict + b_dec) / t_whole / 1e9, 1),
        "algorithmic_bytes_per_step": b_evict + b_dec,
        "pieces_ms": {"evictions_all_layers": round(t_ev * 1e3, 4),
                      "decode_steps_all_layers": round(t_dec * 1e3, 4)},
        "eviction_gbps": round(b_evict / t_ev / 1e9, 1),
        "decode_gbps_cache_resident": round(b_dec / t_dec / 1e9, 1),
        "roofline": {"kernel": "decode over the layers' retained caches (split-K + merge)", "bound": "hbm",
                     "achieved": round(b_dec / t_dec / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(b_dec / t_dec / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": int(b_dec / (S * len(layers)))},
        "cache_flush_before_evictions": flush is not None,
        "decode_steps_as_hip_graph": True,
        "wall_s_timed_loop_incl_flush": round(wall, 4),
        "input_generation_s": round(gen_s, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_snapkv(wl, x, args.cpu_seconds, budgets)
    print(json.dumps(result))


def snapkv_algorithmic_bytes(B, Hq, H, D, n, W, kl, S):
    """Bytes an eviction must move (the window queries, K once, the kept K
    and V rows read and written, the kept ids), those of S decode steps over
    the retained cache (step s attends kl + s + 1 rows of K and V; q in, out
    as fp32), and those of the votes pass (window queries, K once; the votes
    it writes are an intermediate of the eviction and are not counted)."""
    b_evict = B * Hq * W * D * 2 + B * H * n * D * 2 + 2 * 2 * B * H * kl * D * 2 + B * H * kl * 4
    rows_dec = sum(kl + s + 1 for s in range(S))
    b_dec = B * H * rows_dec * 2 * D * 2 + S * (B * Hq * D * 2 + B * Hq * D * 4)
    b_votes = B * Hq * W * D * 2 + B * H * n * D * 2
    return b_evict, b_dec, b_votes


MFMA_BF16_PEAK_TFLOPS = 2500.0


def votes_roofline(b_votes, flops_votes, t_votes, traffic):
    """Roofline of the window x context scoring (row statistics + votes): the
    bound is the one its arithmetic intensity puts it under -- HBM below the
    bf16 ridge (2.5 PFLOP/s / 8 TB/s = 312 flop/B; SnapKV's 32-row window
    over a 32K prompt, 251 flop/B over both passes), the matrix cores above it
    (H2O's 128-row window, 993 flop/B)."""
    intensity = flops_votes / b_votes
    gbps = b_votes / t_votes / 1e9
    tflops = flops_votes / t_votes / 1e12
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    r = {"kernel": "snapkv votes (row statistics + votes, MFMA)", "arithmetic_intensity_flop_per_byte":
         round(intensity, 1), "traffic": traffic, "algorithmic_bytes_per_launch": b_votes,
         "algorithmic_flops_per_launch": flops_votes, "hbm_gbps": round(gbps, 1), "mfma_tflops": round(tflops, 1)}
    if intensity < ridge:
        r.update({"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                  "frac": round(gbps / HBM_PEAK_GBPS, 4)})
    else:
        r.update({"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)})
    return r


def _baseline_workers() -> int:
    """Worker processes for the oracle baseline: the host CPUs this process
    may run on, at most 16 (one GPU's share of a shared host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _run_baseline_pool(fn, shares, seconds):
    """fn(share, seconds) in one spawned worker process per share (the workers
    import numpy and the oracle only, never the GPU); returns their results."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    with ProcessPoolExecutor(max_workers=len(shares), mp_context=multiprocessing.get_context("spawn")) as ex:
        futs = [ex.submit(fn, sh, seconds) for sh in shares]
        return [f.result() for f in futs]


def _snapkv_baseline_worker(units, seconds):
    """One worker of the eviction baseline: the oracle's eviction and decode
    steps on its staged units, cycling through them, on one thread, until
    `seconds` of measured time; returns (units done, seconds measured)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    spent, done = 0.0, 0
    with threadpool_limits(1):
        while spent < seconds:
            u = units[done % len(units)]
            G, W, S, n, R, scale, pool, sink, recent, interval = u["cfg"]
            t0 = time.perf_counter()
            Sv, _, _ = oracle.snapkv_unit_votes(oracle.bf16_to_f64(u["qw"]), oracle.bf16_to_f64(u["k"]), n, scale)
            keep = oracle.eviction_unit_keep(oracle.maxpool1d(Sv, pool), n, W, R, sink, recent, interval)
            kc = np.concatenate([u["k"][keep], u["ks"]])[None]
            vc = np.concatenate([u["v"][keep], u["vs"]])[None]
            for s in range(S):
                oracle.decode_over_rows(u["qs"][s], kc, vc, len(keep) + s + 1, G, scale)
            spent += time.perf_counter() - t0
            done += 1
    return done, spent


def cpu_baseline_snapkv(wl, x, seconds, budgets=None):
    """The oracle's eviction (votes, pool, keep, row copies) and its decode
    steps over the kept rows, per (layer, request, KV head) unit, in one
    single-threaded worker process per host core (at most 16), each timing
    about `seconds` of its own units; the units/s of the workers add up and
    are scaled to the batch."""
    import numpy as np

    from synth import bf16_bits

    G, W, S, n = wl.group, wl.window, wl.decode_steps, wl.prompt
    budgets = budgets or [wl.budget]
    units = [(R, b, g) for R in budgets for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    order = np.random.default_rng(0).permutation(len(units))
    N = min(_baseline_workers(), len(units))
    per = 2 if len(units) >= 2 * N else 1
    interval = wl.interval if wl.interval[1] else None
    shares = [[] for _ in range(N)]
    for i in range(N * per):  # staged before timing: the bf16 bits each unit reads
        R, b, g = units[int(order[i])]
        shares[i % N].append({
            "cfg": (G, W, S, n, R, wl.scale, wl.pool_kernel, wl.sink, wl.recent, interval),
            "qw": bf16_bits(x["q_win"][b, g * G:(g + 1) * G]), "k": bf16_bits(x["k"][b, g]),
            "v": bf16_bits(x["v"][b, g]), "qs": bf16_bits(x["q_steps"][:, b, g * G:(g + 1) * G]),
            "ks": bf16_bits(x["k_steps"][:, b, g]), "vs": bf16_bits(x["v_steps"][:, b, g])})
    res = _run_baseline_pool(_snapkv_baseline_worker, shares, seconds)
    rate = sum(d / t for d, t in res)  # units per second over the workers
    step_s = len(units) / rate
    what = "(layer, request, KV head)" if len(budgets) > 1 else "(request, KV head)"
    return {"value": round(wl.batch * S / step_s, 3), "unit": "tokens/s", "cores": N, "kind": "oracle",
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{sum(d for d, _ in res)} {what} unit evictions ({len(units)} make one step) by {N} "
                      f"single-threaded fp64 numpy worker processes, {N * per} distinct units: votes over the "
                      f"{n}-token prompt, pool, keep, row copies and {S} decode steps each; "
                      f"{sum(t for _, t in res):.1f} s measured in all, the workers' units/s summed and scaled to "
                      f"the batch"}


def copy_calibration(torch):
    """A plain copy of 1 GiB (read 1 GiB, write 1 GiB), run three times: the
    per-dispatch FETCH_SIZE / WRITE_SIZE it reports give the scale from those
    counters to bytes."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4}))


def _quest_baseline_worker(units, seconds):
    """One worker of the decode baseline: builds its units' page summaries with
    the oracle (prefill side, untimed), then times the oracle's decode step
    (bf16 decoding of what it reads, page bounds, KV-head max, selection,
    attention) on them, cycling through units and queries, on one thread,
    until `seconds` of measured time; returns (units done, seconds measured)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    with threadpool_limits(1):
        for u in units:
            P = oracle.pages_of(u["n"])
            u["summ"] = oracle.unit_summaries(oracle.gather_unit_pages(u["k"][:, None], np.arange(P), 0, u["n"]),
                                              u["n"])
        spent, done = 0.0, 0
        while spent < seconds:
            u = units[done % len(units)]
            G, scale, topk, sink, recent, dv = u["cfg"]
            qh = u["q"][(done // len(units)) % len(u["q"])]
            n = u["n"]
            mins, maxs = u["summ"]
            t0 = time.perf_counter()
            qf = oracle.bf16_to_f64(qh)
            if topk > 0:
                A = oracle.unit_kv_head_score(oracle.unit_page_bounds(qf, mins, maxs, scale))
            else:  # forced pages only: nothing is scored
                A = np.zeros(len(mins))
            sel = (oracle.unit_select_forced(A, topk, sink, recent) if sink or recent else oracle.unit_select(A, topk))
            kp = oracle.bf16_to_f64(u["k"])
            vp = kp[..., :dv] if u["v"] is None else oracle.bf16_to_f64(u["v"])
            keys = oracle.unit_selected_tokens(kp, sel, n)
            vals = oracle.unit_selected_tokens(vp, sel, n)
            oracle.unit_attention(qf, keys, vals, scale)
            spent += time.perf_counter() - t0
            done += 1
    return done, spent


def cpu_baseline(wl, x, qs, seconds, topk, sink=0, recent=0):
    """Time the oracle's decode step (page bounds, KV-head scores, selection,
    attention -- given the page summaries, which the oracle builds
    beforehand, untimed -- including the decoding of the bf16 inputs it reads)
    on (request, KV head) units in one single-threaded worker process per host
    core (at most 16), each on two units staged beforehand, cycling through
    the benchmark's queries, for about `seconds`; the workers' units/s add up
    and are scaled to the whole step."""
    import numpy as np

    from synth import bf16_bits

    G = wl.group
    units = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    order = np.random.default_rng(0).permutation(len(units))
    pt = x["page_table"].cpu().numpy()
    lens = x["seq_lens"].cpu().numpy()
    N = min(_baseline_workers(), len(units))
    per = 2 if len(units) >= 2 * N else 1
    nq = min(len(qs), 8)
    qbits = bf16_bits(qs[:nq])
    shares = [[] for _ in range(N)]
    for i in range(N * per):  # staged before timing: the bf16 bits each unit reads
        b, g = units[int(order[i])]
        n = int(lens[b])
        P = -(-n // 16)
        shares[i % N].append({
            "cfg": (G, wl.scale, topk, sink, recent, wl.head_dim_v), "n": n,
            "q": qbits[:, b, g * G:(g + 1) * G],
            "k": torch_index(x["k_pages"], pt[b, :P], g),
            "v": None if x["v_pages"] is None else torch_index(x["v_pages"], pt[b, :P], g)})
    res = _run_baseline_pool(_quest_baseline_worker, shares, seconds)
    rate = sum(d / t for d, t in res)  # units per second over the workers
    step_s = len(units) / rate
    return {"value": round(wl.batch / step_s, 3), "unit": "tokens/s", "cores": N, "kind": "oracle",
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{sum(d for d, _ in res)} (request, KV head) unit steps ({len(units)} make one decode step) "
                      f"by {N} single-threaded fp64 numpy worker processes on {N * per} distinct units and {nq} "
                      f"queries: bf16 decoding of the unit's query and K/V pages, page bounds from the oracle's own "
                      f"page summaries (built untimed), KV-head max, top-k and attention; "
                      f"{sum(t for _, t in res):.1f} s measured in all, the workers' units/s summed and scaled to "
                      f"the step"}


def torch_index(pages, phys, g):
    import numpy as np
    import torch
    from synth import bf16_bits
    idx = torch.from_numpy(np.asarray(phys, dtype=np.int64)).to(pages.device)
    return bf16_bits(pages.index_select(0, idx)[:, g])


if __name__ == "__main__":
    main()
