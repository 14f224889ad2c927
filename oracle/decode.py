"""Oracle: decode with page selection from per-page key bounds — TEST INFRASTRUCTURE.

[SF] §二 and §三-§四: in decoding, a page-level method keeps the whole KV
cache and reads only the pages it selects.  [DMA] §三 mentions keeping a
per-block summary of the cache; here the summary is the element-wise
minimum and maximum key of each page, and a page's score for one query is
the largest q·k any key inside the box [kmin, kmax] can reach:
sum over d of max(q_d * kmin_d, q_d * kmax_d).  Readings taken: a KV
group's score is the sum of its query heads' bounds; the query sits after
every cached token, so no causal mask applies; no page is forced.
"""
from __future__ import annotations

import numpy as np

from .prefill import masked_softmax_attention


def page_minmax(k: np.ndarray, page: int):
    """Element-wise min and max key over each page of `page` tokens.

    k [B,Hkv,L,D] -> kmin, kmax [B,Hkv,L//page,D] (exact: a selection).
    """
    k = np.asarray(k, dtype=np.float64)
    B, H, L, D = k.shape
    n = L // page
    kmin = np.empty((B, H, n, D))
    kmax = np.empty((B, H, n, D))
    for p in range(n):
        blk = k[:, :, p * page:(p + 1) * page, :]
        kmin[:, :, p, :] = blk.min(axis=2)
        kmax[:, :, p, :] = blk.max(axis=2)
    return kmin, kmax


def page_scores(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """s[b, g, p] = sum over heads h of group g, sum over d of
    max(q[b,h,d] * kmin[b,g,p,d], q[b,h,d] * kmax[b,g,p,d]).

    q [B,Hq,D]; kmin/kmax [B,Hkv,nP,D].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = kmin.shape[1]
    G = Hq // Hkv
    s = np.zeros(kmin.shape[:3])
    for b in range(B):
        for g in range(Hkv):
            for h in range(g * G, (g + 1) * G):
                lo = kmin[b, g] * q[b, h][None, :]
                hi = kmax[b, g] * q[b, h][None, :]
                s[b, g] += np.maximum(lo, hi).sum(axis=1)
    return s


def decode_attention(q, k, v, idx, count, page, scale, groups=None):
    """Single-query attention over every token of the selected pages.

    q [B,Hq,D]; k/v [B,Hkv,L,D]; idx [B,Hkv,W] ascending, -1 padded;
    count [B,Hkv].  groups: optional list of (b, g) to evaluate (rest NaN).
    Returns out [B,Hq,D] (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    L = k.shape[2]
    out = np.full((B, Hq, D), np.nan)
    todo = [(b, g) for b in range(B) for g in range(Hkv)] if groups is None else groups
    for (b, g) in todo:
        pages = idx[b, g, :int(count[b, g])]
        keys = np.concatenate([np.arange(p * page, (p + 1) * page) for p in pages]) \
            if len(pages) else np.zeros(0, dtype=np.int64)
        kk = np.asarray(k[b, g], dtype=np.float64)
        vv = np.asarray(v[b, g], dtype=np.float64)
        for h in range(g * G, (g + 1) * G):
            # the query follows all L cached tokens: every key is visible
            o, _ = masked_softmax_attention(q[b, h][None, :], np.array([L]), keys, kk, vv, scale)
            out[b, h] = o[0]
    return out
