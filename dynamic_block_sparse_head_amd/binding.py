"""ctypes binding of libdsa.so: the same entry points as include/dsa.h.

Argument marshalling only.  Tensors are torch tensors on the GPU (torch is
used for device memory and the current HIP stream); every computation runs
in the library's HIP kernels.  There is no fallback: without the built
library, or without a GPU, these functions raise.

The C calls take bare pointers to dense row-major buffers, so every tensor's
full shape is checked here against the sizes derived from the call's
primary input before anything is passed down; a mis-sized tensor raises
ValueError and nothing is launched.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_E_ARG, DSA_E_UNSUPPORTED, DSA_E_WORKSPACE, DSA_E_HIP = 0, -1, -2, -3, -4
DSA_F32, DSA_BF16 = 0, 1
DSA_SCORE_POOLED, DSA_SCORE_PAGE_BOUND, DSA_SCORE_POOLED_HEAD = 0, 1, 2

_c_int, _c_size, _vp, _c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float

# name -> (restype, argtypes); mirrors include/dsa.h
SIGNATURES = {
    "dsa_version": (_c_int, []),
    "dsa_status_string": (ctypes.c_char_p, [_c_int]),
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_block_scores_workspace_size": (_c_size, [_c_int] * 7),
    "dsa_block_scores": (_c_int, [_c_int, _c_int, _vp, _vp, _vp] + [_c_int] * 6
                         + [_vp, _c_size, _vp, _vp]),
    "dsa_topk_select": (_c_int, [_vp] + [_c_int] * 6 + [_vp, _vp, _vp]),
    "dsa_sparse_attn_prefill": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 5 + [_vp, _vp]
                                + [_c_int] * 3 + [_c_float, _vp, _vp, _vp]),
    "dsa_sparse_attn_prefill_backward_workspace_size": (_c_size, [_c_int] * 6),
    "dsa_sparse_attn_prefill_backward": (_c_int, [_c_int] + [_vp] * 4 + [_vp, _vp]
                                         + [_c_int] * 5 + [_vp, _vp] + [_c_int] * 2
                                         + [_c_float, _vp, _c_size, _vp, _vp, _vp, _vp]),
    "dsa_sparse_attn_prefill_ex": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 5 + [_vp, _vp]
                                   + [_c_int] * 3 + [_vp, _c_float, _vp, _vp, _vp]),
    "dsa_dma_weights": (_c_int, [_c_int, _vp] + [_c_int] * 4 + [_vp, _vp, _c_int, _vp, _vp, _vp]),
    "dsa_paged_append": (_c_int, [_c_int, _vp, _vp] + [_c_int] * 5 + [_vp, _vp, _c_int] + [_vp] * 5),
    "dsa_paged_page_scores": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 6
                              + [_vp, _vp, _c_int, _vp, _vp]),
    "dsa_paged_decode": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 6
                         + [_vp, _vp, _c_int, _vp, _vp, _c_int, _c_float, _vp, _c_size, _vp, _vp]),
    "dsa_page_minmax": (_c_int, [_c_int, _vp] + [_c_int] * 5 + [_vp, _vp, _vp]),
    "dsa_sparse_attn_decode_workspace_size": (_c_size, [_c_int] * 6),
    "dsa_sparse_attn_decode": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 5 + [_vp, _vp]
                               + [_c_int] * 2 + [_c_float, _vp, _c_size, _vp, _vp]),
    "dsa_nsa_compress": (_c_int, [_c_int, _vp, _vp] + [_c_int] * 6 + [_vp, _vp, _vp]),
    "dsa_nsa_cmp_attn": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 8
                         + [_c_float, _vp, _vp, _vp, _vp]),
    "dsa_nsa_combine": (_c_int, [_c_int, _vp, _vp, _vp, _vp] + [_c_int] * 4 + [_vp, _vp]),
    "dsa_nsa_cmp_token_scores": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 8
                                 + [_c_float, _vp, _vp]),
    "dsa_topk_select_tokens": (_c_int, [_vp] + [_c_int] * 6 + [_vp, _vp, _vp]),
    "dsa_nsa_window_combine": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 6
                               + [_c_float, _vp, _vp, _vp, _vp, _vp]),
    "dsa_nsa_select_window_combine": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 5 + [_vp, _vp]
                                      + [_c_int] * 3 + [_c_float, _vp, _vp, _vp, _vp]),
    "dsa_sparse_attn_tokens": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 5 + [_vp, _vp]
                               + [_c_int] * 2 + [_c_float, _vp, _vp, _vp]),
    "dsa_sparse_attn_decode_noalloc": (_c_int, [_c_int, _vp, _vp, _vp] + [_c_int] * 5 + [_vp, _vp]
                                       + [_c_int] * 2 + [_c_float, _vp, _vp]),
    "dsa_read_stream_sink_words": (_c_size, []),
    "dsa_read_stream": (_c_int, [_vp, _c_size, _vp, _c_size, _vp]),
}

_lib = None


class DSAError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status}: {message}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa.so once and declare its prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m dynamic_block_sparse_head_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != DSA_OK:
        msg = load().dsa_last_error().decode(errors="replace")
        raise DSAError(status, where, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t, name, dtype=None):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return t.data_ptr()


def _expect(t, shape, name):
    """t must have exactly this shape (None: t is absent and may be None)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")


def _expect_rows(t, lead, last, name):
    """t holds prod(lead) rows of `last` elements: any shape whose trailing
    dimension is `last` (when given) and whose size is prod(lead) * last."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    n = 1
    for x in lead:
        n *= int(x)
    want = n * (1 if last is None else int(last))
    if t.numel() != want or (last is not None and (t.dim() == 0 or t.shape[-1] != last)):
        tail = "" if last is None else f" with last dimension {last}"
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want} elements{tail}")


def _ndim(t, n, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions (got shape {tuple(t.shape)})")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ----------------------------------------------------------------- entries
def dsa_version() -> int:
    return load().dsa_version()


def dsa_block_scores_workspace_size(kind, B, Hq, Hkv, n, D, block) -> int:
    return load().dsa_block_scores_workspace_size(kind, B, Hq, Hkv, n, D, block)


def dsa_block_scores(kind, q, k_or_kmin, kmax, block, workspace, scores, stream=None):
    """POOLED: q [B,Hq,S,D], k [B,Hkv,S,D] -> scores [B,Hkv,nb,nb].
    POOLED_HEAD: the same inputs -> scores [B,Hq,nb,nb] (one per query head).
    PAGE_BOUND: q [B,Hq,D], kmin/kmax [B,Hkv,nP,D] -> scores [B,Hkv,nP]."""
    if kind in (DSA_SCORE_POOLED, DSA_SCORE_POOLED_HEAD):
        _ndim(q, 4, "q")
        _ndim(k_or_kmin, 4, "k")
        B, Hq, n, D = q.shape
        Hkv = k_or_kmin.shape[1]
        _expect(k_or_kmin, (B, Hkv, n, D), "k")
        nb = -(-n // block) if block > 0 else 0
        units = Hkv if kind == DSA_SCORE_POOLED else Hq
        _expect_rows(scores, (B, units, nb), nb, "scores")
    else:
        _ndim(q, 3, "q")
        _ndim(k_or_kmin, 4, "kmin")
        B, Hq, D = q.shape
        Hkv, n = k_or_kmin.shape[1], k_or_kmin.shape[2]
        _expect(k_or_kmin, (B, Hkv, n, D), "kmin")
        _expect(kmax, (B, Hkv, n, D), "kmax")
        _expect_rows(scores, (B, Hkv), n, "scores")
    ws_ptr = _ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().dsa_block_scores(kind, _dtype_code(q), _ptr(q, "q"), _ptr(k_or_kmin, "k"),
                                 _ptr(kmax, "kmax"), B, Hq, Hkv, n, D, block, ws_ptr, ws_bytes,
                                 _ptr(scores, "scores", torch.float32), _stream(stream))
    _check(st, "dsa_block_scores")


def dsa_topk_select(scores, k, n_local, causal, idx, count, stream=None):
    """scores [..., n_q, n_k] float32 -> idx [..., n_q, k+n_local], count [..., n_q] int32."""
    if scores.dim() < 2:
        raise ValueError(f"scores must have at least 2 dimensions (got {tuple(scores.shape)})")
    n_q, n_k = scores.shape[-2], scores.shape[-1]
    rows = scores.numel() // max(1, n_q * n_k)
    _expect_rows(idx, (rows, n_q), k + n_local, "idx")
    _expect_rows(count, (rows, n_q), None, "count")
    st = load().dsa_topk_select(_ptr(scores, "scores", torch.float32), rows, n_q, n_k, k, n_local,
                                int(bool(causal)), _ptr(idx, "idx", torch.int32),
                                _ptr(count, "count", torch.int32), _stream(stream))
    _check(st, "dsa_topk_select")


def _check_attn(q, k, v, out, lse):
    """q, out [B,Hq,S,D]; k, v [B,Hkv,S,D]; lse [B,Hq,S]."""
    _ndim(q, 4, "q")
    _ndim(k, 4, "k")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _expect(k, (B, Hkv, S, D), "k")
    _expect(v, (B, Hkv, S, D), "v")
    _expect(out, (B, Hq, S, D), "out")
    _expect(lse, (B, Hq, S), "lse")
    return B, Hq, Hkv, S, D


def _check_lists(idx, count, units, n_rows, name="idx"):
    """idx [*units, n_rows, width] and count [*units, n_rows]; returns width."""
    if idx is None and count is None:
        return 0
    if idx is None or count is None:
        raise ValueError("idx and count must be given together")
    if idx.dim() < 1:
        raise ValueError(f"{name} must have a last (list) dimension")
    width = idx.shape[-1]
    _expect(idx, (*units, n_rows, width), name)
    _expect(count, (*units, n_rows), "count")
    return width


def dsa_sparse_attn_prefill(q, k, v, idx, count, block, window, scale, out, lse=None, stream=None):
    B, Hq, Hkv, S, D = _check_attn(q, k, v, out, lse)
    nb = -(-S // block) if block > 0 else 0
    width = _check_lists(idx, count, (B, Hkv), nb)
    st = load().dsa_sparse_attn_prefill(
        _dtype_code(q), _ptr(q, "q"), _ptr(k, "k", q.dtype), _ptr(v, "v", q.dtype), B, Hq, Hkv, S, D,
        _ptr(idx, "idx", torch.int32), _ptr(count, "count", torch.int32), width, block, window,
        float(scale), _ptr(out, "out", q.dtype), _ptr(lse, "lse", torch.float32), _stream(stream))
    _check(st, "dsa_sparse_attn_prefill")


def dsa_sparse_attn_prefill_backward_workspace_size(B, Hq, Hkv, S, D, block) -> int:
    return load().dsa_sparse_attn_prefill_backward_workspace_size(B, Hq, Hkv, S, D, block)


def dsa_sparse_attn_prefill_backward(q, k, v, out, lse, dout, idx, count, block, scale, workspace,
                                     dq, dk, dv, stream=None):
    B, Hq, Hkv, S, D = _check_attn(q, k, v, out, lse)
    for t, name in ((dout, "dout"), (dq, "dq")):
        _expect(t, (B, Hq, S, D), name)
    for t, name in ((dk, "dk"), (dv, "dv")):
        _expect(t, (B, Hkv, S, D), name)
    nb = -(-S // block) if block > 0 else 0
    _check_lists(idx, count, (B, Hkv), nb)
    st = load().dsa_sparse_attn_prefill_backward(
        _dtype_code(q), _ptr(q, "q"), _ptr(k, "k", q.dtype), _ptr(v, "v", q.dtype),
        _ptr(out, "out", q.dtype), _ptr(lse, "lse", torch.float32), _ptr(dout, "dout", q.dtype),
        B, Hq, Hkv, S, D, _ptr(idx, "idx", torch.int32), _ptr(count, "count", torch.int32),
        idx.shape[-1], block, float(scale), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(dq, "dq", q.dtype),
        _ptr(dk, "dk", q.dtype), _ptr(dv, "dv", q.dtype), _stream(stream))
    _check(st, "dsa_sparse_attn_prefill_backward")


def dsa_sparse_attn_prefill_ex(q, k, v, idx, count, block, sel_heads, key_bias, scale, out,
                               lse=None, stream=None):
    B, Hq, Hkv, S, D = _check_attn(q, k, v, out, lse)
    nb = -(-S // block) if block > 0 else 0
    if sel_heads < 1 or Hq % sel_heads:
        raise ValueError(f"sel_heads ({sel_heads}) must divide Hq ({Hq})")
    _check_lists(idx, count, (B, Hq // sel_heads), nb)
    _expect(key_bias, (B, Hkv, S), "key_bias")
    st = load().dsa_sparse_attn_prefill_ex(
        _dtype_code(q), _ptr(q, "q"), _ptr(k, "k", q.dtype), _ptr(v, "v", q.dtype), B, Hq, Hkv, S, D,
        _ptr(idx, "idx", torch.int32), _ptr(count, "count", torch.int32), idx.shape[-1], block,
        sel_heads, _ptr(key_bias, "key_bias", torch.float32), float(scale),
        _ptr(out, "out", q.dtype), _ptr(lse, "lse", torch.float32), _stream(stream))
    _check(st, "dsa_sparse_attn_prefill_ex")


def dsa_dma_weights(v, proj, gain, block, weights, block_scores=None, stream=None):
    """v [B,Hkv,S,D] -> weights [B,Hkv,S] (and block_scores [B,Hkv,nb,nb])."""
    _ndim(v, 4, "v")
    B, Hkv, S, D = v.shape
    nb = -(-S // block) if block > 0 else 0
    _expect(proj, (Hkv, D), "proj")
    _expect(gain, (Hkv,), "gain")
    _expect(weights, (B, Hkv, S), "weights")
    _expect(block_scores, (B, Hkv, nb, nb), "block_scores")
    st = load().dsa_dma_weights(_dtype_code(v), _ptr(v, "v"), B, Hkv, S, D,
                                _ptr(proj, "proj", torch.float32), _ptr(gain, "gain", torch.float32),
                                block, _ptr(weights, "weights", torch.float32),
                                _ptr(block_scores, "block_scores", torch.float32), _stream(stream))
    _check(st, "dsa_dma_weights")


def dsa_paged_append(k_new, v_new, page_table, seq_len, k_pool, v_pool, kmin, kmax, stream=None):
    """k_new, v_new [B,Hkv,D]; pools [n_pool,Hkv,page,D]; kmin/kmax [n_pool,Hkv,D];
    page_table [B,max_pages] int32; seq_len [B] int32 (incremented)."""
    _ndim(k_new, 3, "k_new")
    _ndim(k_pool, 4, "k_pool")
    _ndim(page_table, 2, "page_table")
    B, Hkv, D = k_new.shape
    n_pool, _, page, _ = k_pool.shape
    _expect(v_new, (B, Hkv, D), "v_new")
    _expect(k_pool, (n_pool, Hkv, page, D), "k_pool")
    _expect(v_pool, (n_pool, Hkv, page, D), "v_pool")
    _expect(kmin, (n_pool, Hkv, D), "kmin")
    _expect(kmax, (n_pool, Hkv, D), "kmax")
    _expect(page_table, (B, page_table.shape[1]), "page_table")
    _expect(seq_len, (B,), "seq_len")
    st = load().dsa_paged_append(
        _dtype_code(k_new), _ptr(k_new, "k_new"), _ptr(v_new, "v_new", k_new.dtype), B, Hkv, D, page,
        page_table.shape[1], _ptr(page_table, "page_table", torch.int32),
        _ptr(seq_len, "seq_len", torch.int32), n_pool, _ptr(k_pool, "k_pool", k_new.dtype),
        _ptr(v_pool, "v_pool", k_new.dtype), _ptr(kmin, "kmin", k_new.dtype),
        _ptr(kmax, "kmax", k_new.dtype), _stream(stream))
    _check(st, "dsa_paged_append")


def dsa_paged_page_scores(q, kmin, kmax, page, page_table, seq_len, scores, stream=None):
    """q [B,Hq,D]; kmin/kmax [n_pool,Hkv,D] -> scores [B,Hkv,max_pages]."""
    _ndim(q, 3, "q")
    _ndim(kmin, 3, "kmin")
    _ndim(page_table, 2, "page_table")
    B, Hq, D = q.shape
    n_pool, Hkv, _ = kmin.shape
    _expect(kmin, (n_pool, Hkv, D), "kmin")
    _expect(kmax, (n_pool, Hkv, D), "kmax")
    _expect(page_table, (B, page_table.shape[1]), "page_table")
    _expect(seq_len, (B,), "seq_len")
    _expect_rows(scores, (B, Hkv), page_table.shape[1], "scores")
    st = load().dsa_paged_page_scores(
        _dtype_code(q), _ptr(q, "q"), _ptr(kmin, "kmin", q.dtype), _ptr(kmax, "kmax", q.dtype), B, Hq,
        Hkv, D, page, page_table.shape[1], _ptr(page_table, "page_table", torch.int32),
        _ptr(seq_len, "seq_len", torch.int32), n_pool, _ptr(scores, "scores", torch.float32),
        _stream(stream))
    _check(st, "dsa_paged_page_scores")


def dsa_paged_decode(q, k_pool, v_pool, page_table, seq_len, idx, count, scale, workspace, out,
                     stream=None):
    _ndim(q, 3, "q")
    _ndim(k_pool, 4, "k_pool")
    _ndim(page_table, 2, "page_table")
    B, Hq, D = q.shape
    n_pool, Hkv, page, _ = k_pool.shape
    _expect(k_pool, (n_pool, Hkv, page, D), "k_pool")
    _expect(v_pool, (n_pool, Hkv, page, D), "v_pool")
    _expect(page_table, (B, page_table.shape[1]), "page_table")
    _expect(seq_len, (B,), "seq_len")
    _expect_rows(idx, (B, Hkv), idx.shape[-1], "idx")
    _expect_rows(count, (B, Hkv), None, "count")
    _expect(out, (B, Hq, D), "out")
    st = load().dsa_paged_decode(
        _dtype_code(q), _ptr(q, "q"), _ptr(k_pool, "k_pool", q.dtype), _ptr(v_pool, "v_pool", q.dtype),
        B, Hq, Hkv, D, page, page_table.shape[1], _ptr(page_table, "page_table", torch.int32),
        _ptr(seq_len, "seq_len", torch.int32), n_pool, _ptr(idx, "idx", torch.int32),
        _ptr(count, "count", torch.int32), idx.shape[-1], float(scale), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(out, "out", q.dtype), _stream(stream))
    _check(st, "dsa_paged_decode")


def dsa_page_minmax(k, page, kmin, kmax, stream=None):
    _ndim(k, 4, "k")
    B, Hkv, L, D = k.shape
    n_pages = L // page if page > 0 else 0
    _expect_rows(kmin, (B, Hkv, n_pages), D, "kmin")
    _expect_rows(kmax, (B, Hkv, n_pages), D, "kmax")
    st = load().dsa_page_minmax(_dtype_code(k), _ptr(k, "k"), B, Hkv, L, D, page,
                                _ptr(kmin, "kmin", k.dtype), _ptr(kmax, "kmax", k.dtype),
                                _stream(stream))
    _check(st, "dsa_page_minmax")


def dsa_sparse_attn_decode_workspace_size(B, Hq, Hkv, idx_width, page, D) -> int:
    return load().dsa_sparse_attn_decode_workspace_size(B, Hq, Hkv, idx_width, page, D)


def dsa_sparse_attn_decode(q, k_cache, v_cache, idx, count, page, scale, workspace, out,
                           stream=None):
    _ndim(q, 3, "q")
    _ndim(k_cache, 4, "k_cache")
    B, Hq, D = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    _expect(k_cache, (B, Hkv, L, D), "k_cache")
    _expect(v_cache, (B, Hkv, L, D), "v_cache")
    _expect_rows(idx, (B, Hkv), idx.shape[-1], "idx")
    _expect_rows(count, (B, Hkv), None, "count")
    _expect(out, (B, Hq, D), "out")
    st = load().dsa_sparse_attn_decode(
        _dtype_code(q), _ptr(q, "q"), _ptr(k_cache, "k_cache", q.dtype),
        _ptr(v_cache, "v_cache", q.dtype), B, Hq, Hkv, L, D, _ptr(idx, "idx", torch.int32),
        _ptr(count, "count", torch.int32), idx.shape[-1], page, float(scale),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, "out", q.dtype), _stream(stream))
    _check(st, "dsa_sparse_attn_decode")


def dsa_sparse_attn_decode_noalloc(q, k_cache, v_cache, idx, count, page, scale, out,
                                   stream=None):
    """dsa_sparse_attn_decode with the library's per-device scratch in place
    of a workspace (allocates nothing; overlapping calls on one GPU race)."""
    _ndim(q, 3, "q")
    _ndim(k_cache, 4, "k_cache")
    B, Hq, D = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    _expect(k_cache, (B, Hkv, L, D), "k_cache")
    _expect(v_cache, (B, Hkv, L, D), "v_cache")
    _expect_rows(idx, (B, Hkv), idx.shape[-1], "idx")
    _expect_rows(count, (B, Hkv), None, "count")
    _expect(out, (B, Hq, D), "out")
    st = load().dsa_sparse_attn_decode_noalloc(
        _dtype_code(q), _ptr(q, "q"), _ptr(k_cache, "k_cache", q.dtype),
        _ptr(v_cache, "v_cache", q.dtype), B, Hq, Hkv, L, D, _ptr(idx, "idx", torch.int32),
        _ptr(count, "count", torch.int32), idx.shape[-1], page, float(scale),
        _ptr(out, "out", q.dtype), _stream(stream))
    _check(st, "dsa_sparse_attn_decode_noalloc")


def dsa_nsa_compress(k, v, length, stride, ck, cv, stream=None):
    _ndim(k, 4, "k")
    B, Hkv, S, D = k.shape
    n_cmp = (S - length) // stride + 1 if length >= 1 and stride >= 1 and S >= length else 0
    _expect(v, (B, Hkv, S, D), "v")
    _expect(ck, (B, Hkv, n_cmp, D), "ck")
    _expect(cv, (B, Hkv, n_cmp, D), "cv")
    st = load().dsa_nsa_compress(_dtype_code(k), _ptr(k, "k"), _ptr(v, "v", k.dtype), B, Hkv, S, D,
                                 length, stride, _ptr(ck, "ck", k.dtype), _ptr(cv, "cv", k.dtype),
                                 _stream(stream))
    _check(st, "dsa_nsa_compress")


def dsa_nsa_cmp_attn(q, ck, cv, length, stride, sel_block, scale, out, lse, block_scores=None,
                     stream=None):
    _ndim(q, 4, "q")
    _ndim(ck, 4, "ck")
    B, Hq, S, D = q.shape
    Hkv = ck.shape[1]
    n_cmp = (S - length) // stride + 1 if length >= 1 and stride >= 1 and S >= length else 0
    nb = -(-S // sel_block) if sel_block > 0 else 0
    _expect(ck, (B, Hkv, n_cmp, D), "ck")
    _expect(cv, (B, Hkv, n_cmp, D), "cv")
    _expect(out, (B, Hq, S, D), "out")
    _expect(lse, (B, Hq, S), "lse")
    _expect(block_scores, (B, Hkv, nb, nb), "block_scores")
    st = load().dsa_nsa_cmp_attn(
        _dtype_code(q), _ptr(q, "q"), _ptr(ck, "ck", q.dtype), _ptr(cv, "cv", q.dtype), B, Hq, Hkv,
        S, D, length, stride, sel_block, float(scale), _ptr(out, "out", q.dtype),
        _ptr(lse, "lse", torch.float32), _ptr(block_scores, "block_scores", torch.float32),
        _stream(stream))
    _check(st, "dsa_nsa_cmp_attn")


def dsa_nsa_cmp_token_scores(q, ck, lse, length, stride, sel_block, scale, scores, stream=None):
    """Per-token selection scores [B,Hkv,S,nb] from the compressed branch's lse."""
    _ndim(q, 4, "q")
    _ndim(ck, 4, "ck")
    B, Hq, S, D = q.shape
    Hkv = ck.shape[1]
    n_cmp = (S - length) // stride + 1 if length >= 1 and stride >= 1 and S >= length else 0
    nb = -(-S // sel_block) if sel_block > 0 else 0
    _expect(ck, (B, Hkv, n_cmp, D), "ck")
    _expect(lse, (B, Hq, S), "lse")
    _expect(scores, (B, Hkv, S, nb), "scores")
    st = load().dsa_nsa_cmp_token_scores(
        _dtype_code(q), _ptr(q, "q"), _ptr(ck, "ck", q.dtype), _ptr(lse, "lse", torch.float32), B,
        Hq, Hkv, S, D, length, stride, sel_block, float(scale),
        _ptr(scores, "scores", torch.float32), _stream(stream))
    _check(st, "dsa_nsa_cmp_token_scores")


def dsa_topk_select_tokens(scores, k, n_local, block, idx, count, stream=None):
    """scores [..., S, n_k] float32 (one row per token) -> idx [..., S, k+n_local],
    count [..., S] int32; token t's candidates are blocks 0 .. t // block - n_local."""
    if scores.dim() < 2:
        raise ValueError(f"scores must have at least 2 dimensions (got {tuple(scores.shape)})")
    S, n_k = scores.shape[-2], scores.shape[-1]
    rows = scores.numel() // max(1, S * n_k)
    _expect_rows(idx, (rows, S), k + n_local, "idx")
    _expect_rows(count, (rows, S), None, "count")
    st = load().dsa_topk_select_tokens(_ptr(scores, "scores", torch.float32), rows, S, n_k, k,
                                       n_local, block, _ptr(idx, "idx", torch.int32),
                                       _ptr(count, "count", torch.int32), _stream(stream))
    _check(st, "dsa_topk_select_tokens")


def dsa_sparse_attn_tokens(q, k, v, idx, count, block, scale, out, lse=None, stream=None):
    """Selected branch with per-token lists idx [B,Hkv,S,W], count [B,Hkv,S]."""
    B, Hq, Hkv, S, D = _check_attn(q, k, v, out, lse)
    _check_lists(idx, count, (B, Hkv), S)
    st = load().dsa_sparse_attn_tokens(
        _dtype_code(q), _ptr(q, "q"), _ptr(k, "k", q.dtype), _ptr(v, "v", q.dtype), B, Hq, Hkv, S,
        D, _ptr(idx, "idx", torch.int32), _ptr(count, "count", torch.int32), idx.shape[-1], block,
        float(scale), _ptr(out, "out", q.dtype), _ptr(lse, "lse", torch.float32), _stream(stream))
    _check(st, "dsa_sparse_attn_tokens")


def dsa_nsa_window_combine(q, k, v, window, scale, o_cmp, o_sel, gate_logits, out, stream=None):
    """Sliding branch with the gated combine in its epilogue (o_win stays on chip)."""
    B, Hq, Hkv, S, D = _check_attn(q, k, v, out, None)
    _expect(o_cmp, (B, Hq, S, D), "o_cmp")
    _expect(o_sel, (B, Hq, S, D), "o_sel")
    _expect(gate_logits, (B, S, Hq, 3), "gate_logits")
    st = load().dsa_nsa_window_combine(
        _dtype_code(q), _ptr(q, "q"), _ptr(k, "k", q.dtype), _ptr(v, "v", q.dtype), B, Hq, Hkv, S,
        D, window, float(scale), _ptr(o_cmp, "o_cmp", q.dtype), _ptr(o_sel, "o_sel", q.dtype),
        _ptr(gate_logits, "gate_logits", torch.float32), _ptr(out, "out", q.dtype), _stream(stream))
    _check(st, "dsa_nsa_window_combine")


def dsa_nsa_select_window_combine(q, k, v, idx, count, sel_block, window, scale, o_cmp,
                                  gate_logits, out, stream=None):
    """Selected and sliding branches and the gated combine in one pass over
    each query block's rows (o_sel and o_win stay on chip)."""
    B, Hq, Hkv, S, D = _check_attn(q, k, v, out, None)
    nb = -(-S // sel_block) if sel_block > 0 else 0
    width = _check_lists(idx, count, (B, Hkv), nb)
    _expect(o_cmp, (B, Hq, S, D), "o_cmp")
    _expect(gate_logits, (B, S, Hq, 3), "gate_logits")
    st = load().dsa_nsa_select_window_combine(
        _dtype_code(q), _ptr(q, "q"), _ptr(k, "k", q.dtype), _ptr(v, "v", q.dtype), B, Hq, Hkv, S,
        D, _ptr(idx, "idx", torch.int32), _ptr(count, "count", torch.int32), width, sel_block,
        window, float(scale), _ptr(o_cmp, "o_cmp", q.dtype),
        _ptr(gate_logits, "gate_logits", torch.float32), _ptr(out, "out", q.dtype), _stream(stream))
    _check(st, "dsa_nsa_select_window_combine")


def dsa_nsa_combine(o_cmp, o_sel, o_win, gate_logits, out, stream=None):
    _ndim(o_cmp, 4, "o_cmp")
    B, Hq, S, D = o_cmp.shape
    for t, name in ((o_sel, "o_sel"), (o_win, "o_win"), (out, "out")):
        _expect(t, (B, Hq, S, D), name)
    _expect(gate_logits, (B, S, Hq, 3), "gate_logits")
    st = load().dsa_nsa_combine(_dtype_code(o_cmp), _ptr(o_cmp, "o_cmp"),
                                _ptr(o_sel, "o_sel", o_cmp.dtype), _ptr(o_win, "o_win", o_cmp.dtype),
                                _ptr(gate_logits, "gate_logits", torch.float32), B, Hq, S, D,
                                _ptr(out, "out", o_cmp.dtype), _stream(stream))
    _check(st, "dsa_nsa_combine")


def dsa_read_stream(src, sink, stream=None):
    """Read every byte of src once (measurement helper); sink [>= sink words]
    int32 receives one XOR word per workgroup."""
    if not isinstance(src, torch.Tensor) or not isinstance(sink, torch.Tensor):
        raise TypeError("src and sink must be torch.Tensors")
    need = load().dsa_read_stream_sink_words()
    if sink.numel() < need:
        raise ValueError(f"sink has shape {tuple(sink.shape)}, expected at least {need} elements")
    st = load().dsa_read_stream(_ptr(src, "src"), src.numel() * src.element_size(),
                                _ptr(sink, "sink", torch.int32), sink.numel(), _stream(stream))
    _check(st, "dsa_read_stream")
