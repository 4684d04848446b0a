"""Python binding of libse.so, the gfx950 sparse-KV decode library.

Argument marshalling only: every function here has the name of a C entry
point declared in ``include/se.h``, converts tensors to device pointers and the
current torch stream to a ``hipStream_t``, calls the library and raises
``SEError`` on a non-zero status.  All computation happens in the library's
HIP kernels; there is no fallback path.

Tensors passed in must already live on the GPU with the dtypes and layouts
the header documents (bf16 K/V/q, int32 ids and lengths, fp32 outputs).
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libse.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "se.h")

SE_OK, SE_EINVAL, SE_EUNSUPPORTED, SE_EWORKSPACE, SE_EHIP = 0, 1, 2, 3, 4
PAGE_SIZE = 16


class SEError(RuntimeError):
    def __init__(self, status: int, call: str, text: str):
        super().__init__(f"{call} failed: status {status} ({text})")
        self.status = status
        self.call = call


class KvLayout(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("v_is_k_prefix", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("page_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("token_stride", ctypes.c_int64)]


class DecodeParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("head_agg", ctypes.c_int32),
                ("refresh_last_page", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("sink_pages", ctypes.c_int32), ("recent_pages", ctypes.c_int32),
                ("valu_attention", ctypes.c_int32)]


class SnapKVParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_prompt_len", ctypes.c_int32), ("window", ctypes.c_int32),
                ("pool_kernel", ctypes.c_int32), ("budget", ctypes.c_int32),
                ("out_capacity", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("sink", ctypes.c_int32), ("recent", ctypes.c_int32),
                ("interval_begin", ctypes.c_int32), ("interval_end", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIG = {
    "se_version": ([], ctypes.c_int),
    "se_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "se_build_summaries": ([_P, _I, _I, _P, _P, _P, _P, _P], ctypes.c_int),
    "se_sparse_decode_workspace_size": ([_P, _P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "se_sparse_decode": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "se_quest_scores": ([_P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "se_topk_pages": ([_P, _I, _P, _P, _P, _P], ctypes.c_int),
    "se_decode_selected": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "se_sparse_decode_noalloc": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "se_snapkv_workspace_size": ([_P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "se_snapkv_compact": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "se_snapkv_votes": ([_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "se_maxpool1d": ([_P, _P, _P, _P, _P], ctypes.c_int),
    "se_snapkv_select": ([_P, _P, _P, _P, _P, _P], ctypes.c_int),
    "se_compact": ([_P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "se_snapkv_kept_capacity": ([_P, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    "se_snapkv_recompact": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "se_pyramid_budgets": ([_I, _I, ctypes.c_double, ctypes.c_double, ctypes.POINTER(ctypes.c_int32)],
                           ctypes.c_int),
}


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_kv_long_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIG.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


def header_functions() -> list:
    """Names of the functions ``include/se.h`` declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(se_\w+)\s*\(", text, flags=re.M)))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(rc: int, call: str):
    if rc != SE_OK:
        raise SEError(rc, call, lib().se_status_string(rc).decode())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


# ---------------------------------------------------------------------------
# Layout and parameter helpers
# ---------------------------------------------------------------------------
def paged_layout(num_kv_heads: int, head_dim_qk: int, head_dim_v: int, v_is_k_prefix: bool = False) -> KvLayout:
    """Layout of a paged pool [P, Hkv, 16, Dk] (V the same, or inside K)."""
    d = head_dim_qk
    return KvLayout(PAGE_SIZE, num_kv_heads, head_dim_qk, head_dim_v, int(v_is_k_prefix), 0,
                    num_kv_heads * PAGE_SIZE * d, PAGE_SIZE * d, d)


def dense_layout(num_kv_heads: int, capacity: int, head_dim: int) -> KvLayout:
    """Layout of a dense per-request cache [B, Hkv, capacity, D]; page id of
    logical page lp of request b is b*Hkv*capacity/16 + lp."""
    assert capacity % PAGE_SIZE == 0
    return KvLayout(PAGE_SIZE, num_kv_heads, head_dim, head_dim, 0, 0,
                    PAGE_SIZE * head_dim, capacity * head_dim, head_dim)


def decode_params(batch, num_q_heads, max_pages_per_seq, topk, sm_scale=0.0, head_agg=0,
                  refresh_last_page=0, num_splits=0, sink_pages=0, recent_pages=0,
                  valu_attention=0) -> DecodeParams:
    return DecodeParams(batch, num_q_heads, max_pages_per_seq, topk, sm_scale, head_agg, refresh_last_page,
                        num_splits, sink_pages, recent_pages, valu_attention)


def kept_capacity(params: DecodeParams) -> int:
    """Last dimension of `selected` arrays: topk + sink_pages + recent_pages."""
    return params.topk + params.sink_pages + params.recent_pages


def snapkv_params(batch, num_q_heads, num_kv_heads, head_dim, max_prompt_len, window, pool_kernel, budget,
                  out_capacity, sm_scale=0.0, sink=0, recent=0, interval=(0, 0)) -> SnapKVParams:
    return SnapKVParams(batch, num_q_heads, num_kv_heads, head_dim, max_prompt_len, window, pool_kernel, budget,
                        out_capacity, sm_scale, sink, recent, interval[0], interval[1])


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def se_version() -> int:
    return lib().se_version()


def se_status_string(status: int) -> str:
    return lib().se_status_string(status).decode()


def se_build_summaries(layout, batch, max_pages_per_seq, k_pages, page_table, seq_lens, summaries, stream=None):
    _check(lib().se_build_summaries(ctypes.byref(layout), batch, max_pages_per_seq, _ptr(k_pages), _ptr(page_table),
                                    _ptr(seq_lens), _ptr(summaries), _stream(stream)), "se_build_summaries")


def se_sparse_decode_workspace_size(layout, params) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().se_sparse_decode_workspace_size(ctypes.byref(layout), ctypes.byref(params), ctypes.byref(n)),
           "se_sparse_decode_workspace_size")
    return n.value


def se_sparse_decode(layout, params, q, k_pages, v_pages, page_table, summaries, seq_lens, out, selected, workspace,
                     stream=None):
    _check(lib().se_sparse_decode(ctypes.byref(layout), ctypes.byref(params), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                  _ptr(page_table), _ptr(summaries), _ptr(seq_lens), _ptr(out), _ptr(selected),
                                  _ptr(workspace), _nbytes(workspace), _stream(stream)), "se_sparse_decode")


def se_sparse_decode_noalloc(layout, params, q, k_pages, v_pages, page_table, summaries, seq_lens, out, selected,
                             stream=None):
    _check(lib().se_sparse_decode_noalloc(ctypes.byref(layout), ctypes.byref(params), _ptr(q), _ptr(k_pages),
                                          _ptr(v_pages), _ptr(page_table), _ptr(summaries), _ptr(seq_lens), _ptr(out),
                                          _ptr(selected), _stream(stream)), "se_sparse_decode_noalloc")


NOALLOC_SCRATCH_BYTES = 32 << 20  # SE_NOALLOC_SCRATCH_BYTES


def se_quest_scores(layout, params, q, k_pages, page_table, summaries, seq_lens, scores, stream=None):
    _check(lib().se_quest_scores(ctypes.byref(layout), ctypes.byref(params), _ptr(q), _ptr(k_pages), _ptr(page_table),
                                 _ptr(summaries), _ptr(seq_lens), _ptr(scores), _stream(stream)), "se_quest_scores")


def se_topk_pages(params, num_kv_heads, scores, seq_lens, selected, stream=None):
    _check(lib().se_topk_pages(ctypes.byref(params), num_kv_heads, _ptr(scores), _ptr(seq_lens), _ptr(selected),
                               _stream(stream)), "se_topk_pages")


def se_decode_selected(layout, params, q, k_pages, v_pages, page_table, seq_lens, selected, out, workspace,
                       stream=None):
    _check(lib().se_decode_selected(ctypes.byref(layout), ctypes.byref(params), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                    _ptr(page_table), _ptr(seq_lens), _ptr(selected), _ptr(out), _ptr(workspace),
                                    _nbytes(workspace), _stream(stream)), "se_decode_selected")


def se_snapkv_workspace_size(params) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().se_snapkv_workspace_size(ctypes.byref(params), ctypes.byref(n)), "se_snapkv_workspace_size")
    return n.value


def se_snapkv_compact(params, q_win, k, v, prompt_lens, k_out, v_out, kept_idx, kept_len, workspace, stream=None):
    _check(lib().se_snapkv_compact(ctypes.byref(params), _ptr(q_win), _ptr(k), _ptr(v), _ptr(prompt_lens),
                                   _ptr(k_out), _ptr(v_out), _ptr(kept_idx), _ptr(kept_len), _ptr(workspace),
                                   _nbytes(workspace), _stream(stream)), "se_snapkv_compact")


def se_snapkv_kept_capacity(params) -> int:
    n = ctypes.c_int32(0)
    _check(lib().se_snapkv_kept_capacity(ctypes.byref(params), ctypes.byref(n)), "se_snapkv_kept_capacity")
    return n.value


def se_snapkv_recompact(params, q_win, k, v, cache_lens, positions, k_out, v_out, kept_idx, kept_len, workspace,
                        stream=None):
    _check(lib().se_snapkv_recompact(ctypes.byref(params), _ptr(q_win), _ptr(k), _ptr(v), _ptr(cache_lens),
                                     _ptr(positions), _ptr(k_out), _ptr(v_out), _ptr(kept_idx), _ptr(kept_len),
                                     _ptr(workspace), _nbytes(workspace), _stream(stream)), "se_snapkv_recompact")


def se_pyramid_budgets(num_layers, budget, ratio_first, ratio_last) -> list:
    """Host-side arithmetic in the library; returns a list of num_layers ints."""
    out = (ctypes.c_int32 * max(int(num_layers), 1))()
    _check(lib().se_pyramid_budgets(int(num_layers), int(budget), float(ratio_first), float(ratio_last), out),
           "se_pyramid_budgets")
    return list(out)[:int(num_layers)]


def se_snapkv_votes(params, q_win, k, prompt_lens, votes, workspace, stream=None):
    _check(lib().se_snapkv_votes(ctypes.byref(params), _ptr(q_win), _ptr(k), _ptr(prompt_lens), _ptr(votes),
                                 _ptr(workspace), _nbytes(workspace), _stream(stream)), "se_snapkv_votes")


def se_maxpool1d(params, votes, prompt_lens, pooled, stream=None):
    _check(lib().se_maxpool1d(ctypes.byref(params), _ptr(votes), _ptr(prompt_lens), _ptr(pooled), _stream(stream)),
           "se_maxpool1d")


def se_snapkv_select(params, pooled, prompt_lens, kept_idx, kept_len, stream=None):
    _check(lib().se_snapkv_select(ctypes.byref(params), _ptr(pooled), _ptr(prompt_lens), _ptr(kept_idx),
                                  _ptr(kept_len), _stream(stream)), "se_snapkv_select")


def se_compact(params, k, v, kept_idx, kept_len, k_out, v_out, stream=None):
    _check(lib().se_compact(ctypes.byref(params), _ptr(k), _ptr(v), _ptr(kept_idx), _ptr(kept_len), _ptr(k_out),
                            _ptr(v_out), _stream(stream)), "se_compact")
