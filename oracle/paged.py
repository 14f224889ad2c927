"""Oracle: decode over a paged KV cache — TEST INFRASTRUCTURE.

[SF] §二-§四: a page-level decode method keeps the whole KV cache and reads
only the pages it selects; serving keeps every sequence's cache as pages of
one shared pool.  This module states that computation for a pool
k_pool, v_pool [P, Hkv, page, D] shared by a batch of sequences of different
lengths: page_table[b, p] names the pool page holding tokens
p*page .. p*page+page-1 of sequence b, seq_len[b] counts its tokens (the
last page may be partly filled).  Readings taken: a page's min/max summary
covers only the sequence's tokens written so far (updated as tokens are
appended); pages past a sequence's length score -inf and hold nothing;
otherwise the contiguous decode path's readings hold (group score = sum of
the heads' bounds, no page forced, no causal mask for the query).
"""
from __future__ import annotations

import numpy as np

from .decode import page_scores as dense_page_scores
from .prefill import masked_softmax_attention


def n_pages(seq_len, page):
    return -(-np.asarray(seq_len) // page)


def append(k_pool, v_pool, kmin, kmax, page_table, seq_len, k_new, v_new):
    """Write token seq_len[b] of every sequence b (k_new, v_new [B,Hkv,D])
    into its page and fold its key into that page's min/max (a page's first
    token sets them).  Returns updated copies and seq_len + 1."""
    k_pool, v_pool = k_pool.copy(), v_pool.copy()
    kmin, kmax = kmin.copy(), kmax.copy()
    page = k_pool.shape[2]
    for b in range(k_new.shape[0]):
        t = int(seq_len[b])
        phys = int(page_table[b, t // page])
        r = t % page
        k_pool[phys, :, r] = k_new[b]
        v_pool[phys, :, r] = v_new[b]
        if r == 0:
            kmin[phys] = k_new[b]
            kmax[phys] = k_new[b]
        else:
            kmin[phys] = np.minimum(kmin[phys], k_new[b])
            kmax[phys] = np.maximum(kmax[phys], k_new[b])
    return k_pool, v_pool, kmin, kmax, np.asarray(seq_len) + 1


def gather(pool, page_table, seq_len, b, page):
    """Sequence b's tokens [Hkv, seq_len[b], D] read through its page table."""
    n = int(seq_len[b])
    pages = [pool[int(page_table[b, p])] for p in range(int(n_pages(n, page)))]
    if not pages:
        return np.zeros((pool.shape[1], 0, pool.shape[3]))
    return np.concatenate(pages, axis=1)[:, :n]


def page_scores(q, kmin, kmax, page_table, seq_len, page):
    """s[b, g, p] = the page bound score of logical page p of sequence b
    (its pool page's summary), -inf for p >= ceil(seq_len[b] / page).
    q [B,Hq,D]; kmin/kmax [P,Hkv,D]; -> [B,Hkv,max_pages]."""
    q = np.asarray(q, dtype=np.float64)
    B = q.shape[0]
    Hkv = kmin.shape[1]
    max_pages = page_table.shape[1]
    s = np.full((B, Hkv, max_pages), -np.inf)
    for b in range(B):
        npg = int(n_pages(seq_len[b], page))
        if npg == 0:
            continue
        phys = page_table[b, :npg]
        lo = np.asarray(kmin, dtype=np.float64)[phys].transpose(1, 0, 2)[None]   # [1,Hkv,npg,D]
        hi = np.asarray(kmax, dtype=np.float64)[phys].transpose(1, 0, 2)[None]
        s[b, :, :npg] = dense_page_scores(q[b:b + 1], lo, hi)[0]
    return s


def decode(q, k_pool, v_pool, page_table, seq_len, idx, count, scale):
    """Single-query attention over the tokens (below seq_len) of the selected
    logical pages; selected pages past the sequence's length hold nothing.
    q [B,Hq,D]; idx [B,Hkv,W] (ascending, -1 padded), count [B,Hkv].
    Returns out [B,Hq,D] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    page = k_pool.shape[2]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(seq_len[b])
        kk = np.asarray(gather(k_pool, page_table, seq_len, b, page), dtype=np.float64)
        vv = np.asarray(gather(v_pool, page_table, seq_len, b, page), dtype=np.float64)
        for g in range(Hkv):
            pages = [int(p) for p in idx[b, g, :int(count[b, g])] if 0 <= p < n_pages(n, page)]
            keys = np.concatenate([np.arange(p * page, min((p + 1) * page, n)) for p in pages]) \
                if pages else np.zeros(0, dtype=np.int64)
            for h in range(g * G, (g + 1) * G):
                o, _ = masked_softmax_attention(q[b, h][None, :], np.array([n]), keys, kk[g], vv[g],
                                                scale)
                out[b, h] = o[0]
    return out
