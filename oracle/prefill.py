"""Oracle: causal top-k block-sparse prefill — TEST INFRASTRUCTURE.

Follows [DMA] §四 and §五: score every history position (here: every key
block, scored against each query block), apply the causal mask, keep the
k best-scoring history blocks and set everything else to minus infinity,
then run exact softmax attention over the kept positions only.  [SA]
"策略" (block-sparse pattern: dense inside a block, sparse between blocks)
and [SF] §二 (unit of sparsification = blocks, dynamic content-aware
importance, uniform budget) fix the block granularity.  Readings taken where
the pages are silent:
  * selection unit under grouped-query attention: the KV head; the group's
    block score is the sum of its query heads' scores (`sel_heads`, the
    number of query heads sharing one selection, defaults to the group size;
    sel_heads = 1 is the per-query-head variant: every head ranks blocks by
    its own score and keeps its own list);
  * block score: mean-pooled query block · mean-pooled key block, no 1/sqrt(D);
  * the local window is the n_local most recent key blocks (diagonal
    included); top-k is drawn from the blocks before the window;
  * ties rank the lower block index first; NaN ranks last;
  * index rows are ascending, padded with -1; softmax scale 1/sqrt(D).
"""
from __future__ import annotations

import math

import numpy as np


def pool_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of each run of `block` rows along axis -2 (last run may be short).

    x [..., S, D] -> [..., ceil(S/block), D].  [SA] "策略": a block is a
    contiguous run of positions; its summary here is the plain mean.
    """
    x = np.asarray(x, dtype=np.float64)
    S = x.shape[-2]
    n = -(-S // block)
    out = np.empty(x.shape[:-2] + (n, x.shape[-1]), dtype=np.float64)
    for j in range(n):
        out[..., j, :] = x[..., j * block:min((j + 1) * block, S), :].mean(axis=-2)
    return out


def _units(Hq: int, Hkv: int, sel_heads):
    """(heads per selection unit, number of units per sequence)."""
    G = Hq // Hkv
    u = G if sel_heads is None else int(sel_heads)
    if u < 1 or G % u:
        raise ValueError(f"sel_heads {u} must divide the group size {G}")
    return u, Hq // u


def block_scores_pooled(q: np.ndarray, k: np.ndarray, block: int, sel_heads=None) -> np.ndarray:
    """Block scores s[b, u, i, j] for key block j against query block i, per
    selection unit u (sel_heads consecutive query heads; default: the KV group).

    s = sum over the query heads h of unit u of qbar[b,h,i] · kbar[b,g,j],
    with g the KV head of those query heads; defined for j <= i (causal,
    [DMA] §五: causal mask before top-k); entries j > i are -inf.
    q [B,Hq,S,D], k [B,Hkv,S,D] -> [B, Hq/sel_heads, nb, nb].
    """
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    uh, U = _units(Hq, Hkv, sel_heads)
    qbar = pool_blocks(q, block)
    kbar = pool_blocks(k, block)
    n = qbar.shape[-2]
    s = np.full((B, U, n, n), -np.inf)
    for b in range(B):
        for u in range(U):
            g = (u * uh) // G
            for i in range(n):
                acc = np.zeros(i + 1)
                for h in range(u * uh, (u + 1) * uh):
                    acc += kbar[b, g, :i + 1, :] @ qbar[b, h, i, :]
                s[b, u, i, :i + 1] = acc
    return s


def _rank_key(score: float, j: int):
    # Higher score first, then lower index; NaN after every number.
    return (1, 0.0, j) if math.isnan(score) else (0, -score, j)


def select_blocks(scores: np.ndarray, k: int, n_local: int, causal: bool, row_block: int = 1):
    """Top-k selection plus the local window, per score row.

    scores [..., nQ, nK].  For row r (causal) with i = r // row_block (rows
    are query blocks when row_block = 1, tokens of `row_block`-token blocks
    otherwise): candidates are key blocks 0 .. i - n_local, the window is
    blocks max(0, i-n_local+1) .. i.
    Non-causal rows (decode, one row per group): candidates are blocks
    0 .. nK-1-n_local, the window is the last n_local blocks.
    Candidates are ordered by (score descending, index ascending) and the
    first k kept ([DMA] §五: keep the k highest-weight history positions,
    the rest become -inf).  Output: idx [..., nQ, k + n_local] int32,
    ascending, padded with -1; count [..., nQ] int32.
    """
    scores = np.asarray(scores, dtype=np.float64)
    lead = scores.shape[:-2]
    nQ, nK = scores.shape[-2:]
    width = k + n_local
    idx = np.full(lead + (nQ, width), -1, dtype=np.int32)
    cnt = np.zeros(lead + (nQ,), dtype=np.int32)
    for pos in np.ndindex(*lead) if lead else [()]:
        for r in range(nQ):
            row = scores[pos + (r,)]
            i = r // row_block
            if causal:
                last = i - n_local
                window = list(range(max(0, i - n_local + 1), i + 1))
            else:
                last = nK - 1 - n_local
                window = list(range(nK - n_local, nK))
            cands = list(range(0, last + 1))
            if len(cands) > k:
                cands.sort(key=lambda j: _rank_key(float(row[j]), j))
                cands = cands[:k]
            chosen = sorted(set(cands) | set(window))
            idx[pos + (r,)][:len(chosen)] = chosen
            cnt[pos + (r,)] = len(chosen)
    return idx, cnt


def visible_keys(sel_row: np.ndarray, count: int, block: int, S: int) -> np.ndarray:
    """Token positions covered by the selected key blocks, ascending."""
    toks = [np.arange(j * block, min((j + 1) * block, S)) for j in sel_row[:count]]
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def masked_softmax_attention(q_rows, t_rows, keys, k, v, scale):
    """Exact softmax attention of query rows at positions t_rows over key
    positions `keys`, each row seeing only keys s <= t ([DMA] §四-§五:
    masked positions get weight exactly zero and are never multiplied).

    Returns (out [R,D], lse [R]); a row with no visible key gets out = 0 and
    lse = -inf.
    """
    R = q_rows.shape[0]
    D = v.shape[-1]
    out = np.zeros((R, D))
    lse = np.full(R, -np.inf)
    if keys.size == 0:
        return out, lse
    logits = (q_rows @ k[keys].T) * scale
    visible = keys[None, :] <= t_rows[:, None]
    logits = np.where(visible, logits, -np.inf)
    for r in range(R):
        if not visible[r].any():
            continue
        m = logits[r].max()
        p = np.exp(logits[r] - m)
        l = p.sum()
        out[r] = (p @ v[keys]) / l
        lse[r] = m + math.log(l)
    return out, lse


def sparse_attention(q, k, v, idx, count, block, scale, q_blocks=None, sel_heads=None):
    """Block-sparse causal attention over the selected key blocks.

    q [B,Hq,S,D], k/v [B,Hkv,S,D]; idx [B,U,nB,W] (ascending, -1 padded),
    count [B,U,nB] with U = Hq / sel_heads selection units (default: one per
    KV group).  Query head h uses the index rows of unit h // sel_heads and
    the K/V of its group.  Row t of query block i attends to keys s <= t
    lying in the selected blocks of row i.  q_blocks: optional list of query
    blocks to evaluate (others are left as NaN), for sampled checks at full
    size.  Returns out [B,Hq,S,D], lse [B,Hq,S] (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    uh, _ = _units(Hq, Hkv, sel_heads)
    n = -(-S // block)
    blocks = range(n) if q_blocks is None else q_blocks
    out = np.full((B, Hq, S, v.shape[-1]), np.nan)   # value width may differ from D
    lse = np.full((B, Hq, S), np.nan)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            u = h // uh
            for i in blocks:
                t = np.arange(i * block, min((i + 1) * block, S))
                keys = visible_keys(idx[b, u, i], int(count[b, u, i]), block, S)
                o, l = masked_softmax_attention(q[b, h, t], t, keys, k[b, g], v[b, g], scale)
                out[b, h, t] = o
                lse[b, h, t] = l
    return out, lse


def prefill(q, k, v, block, topk, n_local, scale, sel_heads=None):
    """The whole prefill path: pooled scores -> selection -> attention."""
    s = block_scores_pooled(q, k, block, sel_heads)
    idx, cnt = select_blocks(s, topk, n_local, causal=True)
    out, lse = sparse_attention(q, k, v, idx, cnt, block, scale, sel_heads=sel_heads)
    return {"scores": s, "idx": idx, "count": cnt, "out": out, "lse": lse}
