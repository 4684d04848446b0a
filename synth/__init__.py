"""Seeded synthetic inputs for sparse-KV decode and SnapKV eviction.

This module only draws data: shapes, seeded random values and their rounding
to bf16.  It holds none of the method's arithmetic (no summaries, scores,
selection or attention), so both the HIP path and the CPU oracle may take their
inputs from it without sharing any computation.

Shapes follow the workloads measured on the SparseEngine pages (Fig. 5-8:
128K- and 32K-token inputs on Qwen3-30B-A3B and GLM-4.7-Flash, Quest with
16-token pages, SnapKV with a 32-token scoring window and pooling kernel 7,
Table 8).  The pages publish no data; every value here is synthetic.

Layouts (all bf16 tensors are ``torch.bfloat16``; ids are ``torch.int32``):

* ``q``           [B, Hq, Dk]
* ``k_pages``     [P, Hkv, 16, Dk]   physical page pool, one 16-token page per row
* ``v_pages``     [P, Hkv, 16, Dv]   (``None`` when V is the first Dv dims of K)
* ``page_table``  [B, max_pages]     logical page -> physical page
* ``seq_lens``    [B]                tokens per request (counts the current token)

Physical pages are a seeded permutation of the pool, so the page table really
is an indirection.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

PAGE = 16
BF16_NAN = 0x7FC0


@dataclasses.dataclass(frozen=True)
class QuestWorkload:
    """A Quest decode workload: one attention layer's decode step for a batch."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    context: int  # tokens per request (upper bound when ``ragged_lo`` is set)
    topk: int  # pages kept per (request, KV head)
    saliency: str  # "none" | "heavy" | "outlier" | "zipf"
    v_is_k_prefix: bool = False
    ragged_lo: int = 0  # >0: lengths uniform in [ragged_lo, context]
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_pages(self) -> int:
        return (self.context + PAGE - 1) // PAGE

    @property
    def scale(self) -> float:
        # 1/sqrt(Dk) rounded to fp32, the value both sides are handed
        return float(torch.tensor(1.0 / math.sqrt(self.head_dim_qk), dtype=torch.float32))

    def resized(self, **kw) -> "QuestWorkload":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class SnapKVWorkload:
    """SnapKV prefill eviction followed by dense decode over the retained cache."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    prompt: int
    window: int
    pool_kernel: int
    budget: int
    decode_steps: int
    seed: int = 0
    ragged_lo: int = 0
    method: str = "SnapKV"
    sink: int = 0                 # leading tokens always kept
    recent: int = 0               # trailing tokens always kept (at least the window)
    interval: tuple = (0, 0)      # history span that may be pruned; (0, 0): the whole prompt
    layers: int = 1               # layers evicted per prefill (PyramidKV: one budget per layer)
    layer_ratios: tuple = (1.0, 1.0)  # PyramidKV's first and last layer ratios

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.head_dim), dtype=torch.float32))

    @property
    def out_capacity(self) -> int:
        # for the plain SnapKV shapes (no sink, recent or interval)
        # kept rows plus room for the decode steps, rounded up to whole pages
        need = self.budget + self.window + self.decode_steps
        return (need + PAGE - 1) // PAGE * PAGE

    def resized(self, **kw) -> "SnapKVWorkload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Shapes are those of the models and inputs named on the
# pages; the value distributions are stated in the design notes.
TINY_QUEST = QuestWorkload("tiny_quest_4k", 1, 4, 1, 64, 64, 4096, 32, "heavy", seed=1001)
QWEN3_4B_32K = QuestWorkload("gqa32x8_d128_32k_b8", 8, 32, 8, 128, 128, 32768, 128, "outlier", seed=1002)
QWEN3_30B_128K = QuestWorkload("gqa32x4_d128_128k_b32", 32, 32, 4, 128, 128, 131072, 256, "zipf", seed=1003)
SNAPKV_32K = SnapKVWorkload("snapkv_gqa32x8_d128_32k_b16", 16, 32, 8, 128, 32768, 32, 7, 2048, 64, seed=1004)
# Eviction-family legs on the SnapKV workload's shape and values (same seed):
# H2O with Table 8's settings (8,192 prefill tokens split by the recent ratio
# 0.5, a 128-token scoring window, no pooling), and prefix-cache pruning
# (Figure 4) of a 24K-token history span [4096, 28672) to 2048 tokens.
H2O_32K = SnapKVWorkload("h2o_gqa32x8_d128_32k_b16", 16, 32, 8, 128, 32768, 128, 1, 4096, 64, seed=1004,
                         method="H2O", recent=4096)
PRUNE_32K = SnapKVWorkload("prune_gqa32x8_d128_32k_b16", 16, 32, 8, 128, 32768, 32, 7, 2048, 64, seed=1004,
                           method="prefix-cache pruning", interval=(4096, 28672))
# PyramidKV with Table 8's settings (sink 64, recent 512, 4,096 selected on
# average, layer ratios 0.6 to 0.01, 32-token window; pooling 7 as SnapKV) over
# a 4-layer slice of the stack; every layer sees the same synthetic cache.
PYRAMID_32K = SnapKVWorkload("pyramid4_gqa32x8_d128_32k_b16", 16, 32, 8, 128, 32768, 32, 7, 4096, 64, seed=1004,
                             method="PyramidKV", sink=64, recent=512, layers=4, layer_ratios=(0.6, 0.01))
MLA_RAGGED = QuestWorkload("mla576_h32_ragged16k-128k_b16", 16, 32, 1, 576, 512, 131072, 256, "none",
                           v_is_k_prefix=True, ragged_lo=16384, seed=1005)

WORKLOADS = {w.name: w for w in (TINY_QUEST, QWEN3_4B_32K, QWEN3_30B_128K, SNAPKV_32K, MLA_RAGGED, H2O_32K,
                                 PRUNE_32K, PYRAMID_32K)}


def _gen(device, seed: int, tag: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tag * 7_919) % (2**63 - 1))
    return g


def _randn(shape, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def zipf_magnitudes(n: int, s: float = 1.1) -> torch.Tensor:
    """m_r = sqrt(n * r^-s / H_{n,s}) for ranks r = 1..n, so that mean(m^2) = 1."""
    r = torch.arange(1, n + 1, dtype=torch.float64)
    w = r.pow(-s)
    return torch.sqrt(n * w / w.sum()).to(torch.float32)


def make_quest_inputs(wl: QuestWorkload, device="cpu", poison_tail: bool = False,
                      seq_lens: Optional[list] = None, pool_extra: int = 0) -> dict:
    """Draw one decode step's inputs for ``wl`` on ``device``.

    ``poison_tail`` writes bf16 NaN into the unused slots of each request's
    last page, so a reader that touches tokens past ``seq_lens`` shows up.
    ``seq_lens`` overrides the drawn lengths (each must be <= ``wl.context``).
    """
    dev = torch.device(device)
    B, Hq, Hkv, Dk, Dv = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim_qk, wl.head_dim_v
    G, MP = wl.group, wl.max_pages
    seed = wl.seed

    if seq_lens is not None:
        lens = torch.tensor(seq_lens, dtype=torch.int32)
        assert lens.numel() == B and int(lens.max()) <= wl.context
    elif wl.ragged_lo:
        lens = torch.randint(wl.ragged_lo, wl.context + 1, (B,), generator=_gen("cpu", seed, 1),
                             dtype=torch.int64).to(torch.int32)
    else:
        lens = torch.full((B,), wl.context, dtype=torch.int32)

    pool = B * MP + pool_extra
    perm = torch.randperm(pool, generator=_gen("cpu", seed, 2)).to(torch.int32)
    page_table = perm[: B * MP].reshape(B, MP).contiguous()

    q32 = _randn((B, Hq, Dk), _gen(dev, seed, 3), dev)
    q = q32.to(torch.bfloat16)

    k_pages = torch.empty((pool, Hkv, PAGE, Dk), dtype=torch.bfloat16, device=dev)
    v_pages = None if wl.v_is_k_prefix else torch.empty((pool, Hkv, PAGE, Dv), dtype=torch.bfloat16, device=dev)
    if pool_extra:
        unused = perm[B * MP:].to(dev, torch.int64)
        k_pages[unused] = _randn((pool_extra, Hkv, PAGE, Dk), _gen(dev, seed, 4), dev).to(torch.bfloat16)
        if v_pages is not None:
            v_pages[unused] = _randn((pool_extra, Hkv, PAGE, Dv), _gen(dev, seed, 5), dev).to(torch.bfloat16)

    outlier_ch = None
    if wl.saliency == "outlier":
        outlier_ch = torch.randperm(Dk, generator=_gen("cpu", seed, 6))[:4].to(dev)
    zipf = zipf_magnitudes(MP * PAGE).to(dev) if wl.saliency == "zipf" else None

    for b in range(B):
        kz = _randn((MP, Hkv, PAGE, Dk), _gen(dev, seed, 100 + b), dev)
        if wl.saliency == "outlier":
            kz[..., outlier_ch] *= 8.0
        elif wl.saliency == "zipf":
            for g in range(Hkv):
                ranks = torch.randperm(MP * PAGE, generator=_gen(dev, seed, 10_000 + b * Hkv + g), device=dev)
                kz[:, g] *= zipf[ranks].reshape(MP, PAGE, 1)
        elif wl.saliency == "heavy":
            n = int(lens[b])
            for g in range(Hkv):
                qbar = q[b, g * G:(g + 1) * G].float().mean(0)
                pos = torch.randperm(n, generator=_gen("cpu", seed, 20_000 + b * Hkv + g))[:8]
                for t in pos.tolist():
                    kz[t // PAGE, g, t % PAGE] = 4.0 * qbar
        rows = page_table[b].to(dev, torch.int64)
        k_pages[rows] = kz.to(torch.bfloat16)
        del kz
        if v_pages is not None:
            vz = _randn((MP, Hkv, PAGE, Dv), _gen(dev, seed, 200_000 + b), dev)
            if wl.saliency == "outlier":
                vz[..., outlier_ch] *= 8.0
            v_pages[rows] = vz.to(torch.bfloat16)
            del vz

    if poison_tail:
        nan = torch.tensor(BF16_NAN, dtype=torch.int16).view(torch.bfloat16).to(dev)
        for b in range(B):
            n = int(lens[b])
            if n % PAGE and n > 0:
                lp = n // PAGE
                phys = int(page_table[b, lp])
                k_pages[phys, :, n % PAGE:] = nan
                if v_pages is not None:
                    v_pages[phys, :, n % PAGE:] = nan

    return {
        "q": q,
        "k_pages": k_pages,
        "v_pages": v_pages,
        "page_table": page_table.to(dev),
        "seq_lens": lens.to(dev),
        "scale": wl.scale,
        "topk": wl.topk,
        "group": G,
    }


def make_snapkv_inputs(wl: SnapKVWorkload, device="cpu", prompt_lens: Optional[list] = None,
                       with_decode: bool = True) -> dict:
    """Draw a SnapKV prefill (window queries, K, V) and the decode steps after it."""
    dev = torch.device(device)
    B, Hq, Hkv, D, N, W = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.prompt, wl.window
    seed = wl.seed
    if prompt_lens is not None:
        lens = torch.tensor(prompt_lens, dtype=torch.int32)
        assert lens.numel() == B and int(lens.max()) <= N
    elif wl.ragged_lo:
        lens = torch.randint(wl.ragged_lo, N + 1, (B,), generator=_gen("cpu", seed, 1), dtype=torch.int64).to(torch.int32)
    else:
        lens = torch.full((B,), N, dtype=torch.int32)
    q_win = _randn((B, Hq, W, D), _gen(dev, seed, 3), dev).to(torch.bfloat16)
    k = torch.empty((B, Hkv, N, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty((B, Hkv, N, D), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        k[b] = _randn((Hkv, N, D), _gen(dev, seed, 100 + b), dev).to(torch.bfloat16)
        v[b] = _randn((Hkv, N, D), _gen(dev, seed, 200_000 + b), dev).to(torch.bfloat16)
    out = {"q_win": q_win, "k": k, "v": v, "prompt_lens": lens.to(dev), "scale": wl.scale}
    if with_decode:
        S = wl.decode_steps
        out["q_steps"] = _randn((S, B, Hq, D), _gen(dev, seed, 7), dev).to(torch.bfloat16)
        out["k_steps"] = _randn((S, B, Hkv, D), _gen(dev, seed, 8), dev).to(torch.bfloat16)
        out["v_steps"] = _randn((S, B, Hkv, D), _gen(dev, seed, 9), dev).to(torch.bfloat16)
    return out


def bf16_bits(t: torch.Tensor):
    """The raw bf16 bit patterns of ``t`` as a host numpy uint16 array."""
    import numpy as np
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
