"""The oracle on one (request, KV head) unit per call, run in worker processes.

TEST INFRASTRUCTURE for the full-size parity tests: the oracle is plain
single-threaded numpy with Python loops over pages, so comparing every unit
of a 128K-context batch takes minutes on one core.  These workers are started
with the spawn method and import numpy and the oracle only -- never torch or
the GPU library; the test process fetches each unit's bf16 bits from the GPU
and hands them over.
"""
from __future__ import annotations

import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

import oracle


def workers() -> int:
    """Worker count: the CPUs this process may run on, at most 8."""
    return max(1, min(8, len(os.sched_getaffinity(0))))


def pool() -> ProcessPoolExecutor:
    return ProcessPoolExecutor(max_workers=workers(), mp_context=multiprocessing.get_context("spawn"))


def map_bounded(ex, fn, jobs, depth=None):
    """Submit fn(*args) for each args in the iterable `jobs` (built lazily, so
    at most `depth` units' inputs are alive at once) and yield (key, result)
    in submission order; each job is (key, args)."""
    depth = depth or 2 * workers()
    pending = []
    for key, args in jobs:
        pending.append((key, ex.submit(fn, *args)))
        if len(pending) >= depth:
            k, f = pending.pop(0)
            yield k, f.result()
    for k, f in pending:
        yield k, f.result()


def quest_unit(kbits, vbits_chosen, q_bits, n, scale, chosen, dv, v_is_k_prefix):
    """O1-O3 and O5 for one unit.

    kbits: bf16 bits [P, 16, Dk] of the unit's logical pages (P = ceil(n/16));
    vbits_chosen: bf16 bits [len(chosen), 16, Dv] of the chosen pages' values
    (None when V is the first Dv channels of K); q_bits: [G, Dk]; chosen: the
    logical page ids whose tokens the attention reads (the GPU's selection).
    Returns (mins, maxs, A, out): the page summaries, the KV-head page scores
    and the attention output over the chosen pages.
    """
    P = oracle.pages_of(n)
    kp = oracle.gather_unit_pages(kbits[:, None], np.arange(P), 0, n)
    mins, maxs = oracle.unit_summaries(kp, n)
    qf = oracle.bf16_to_f64(q_bits)
    A = oracle.unit_kv_head_score(oracle.unit_page_bounds(qf, mins, maxs, scale))
    chosen = np.asarray(chosen, dtype=np.int64)
    keys = oracle.unit_selected_tokens(kp, chosen, n)
    if v_is_k_prefix:
        vals = keys[:, :dv]
    else:
        vp = np.full((P, 16, dv), np.nan)
        vp[chosen] = oracle.bf16_to_f64(vbits_chosen)
        tail = n - (P - 1) * 16
        if tail < 16:
            vp[P - 1, tail:] = np.nan  # slots past the last token are never read
        vals = oracle.unit_selected_tokens(vp, chosen, n)
    out = oracle.unit_attention(qf, keys, vals, scale)
    return mins, maxs, A, out, float(np.abs(vals).max()) if vals.size else 0.0


def snapkv_unit(q_bits, k_bits, n, scale, pool_kernel):
    """O6's pooled votes of one unit: q_bits [G, W, D], k_bits [>=n, D]."""
    S, _, _ = oracle.snapkv_unit_votes(oracle.bf16_to_f64(q_bits), oracle.bf16_to_f64(k_bits), n, scale)
    return oracle.maxpool1d(S, pool_kernel)


def decode_rows(q_bits, k_bits, v_bits, length, group, scale):
    """O7: one decode step of one request over its retained rows."""
    return oracle.decode_over_rows(q_bits, k_bits, v_bits, length, group, scale)
