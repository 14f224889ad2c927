"""Oracle: three-branch gated attention — TEST INFRASTRUCTURE.

[NSA] §03: three attention branches run side by side over the same causal
history — (1) compressed: a coarse pass over summaries of the history,
(2) selected: attention over the important blocks only, (3) sliding: the
local context — and a small per-token gate turns each token's context into
three weights that combine the three outputs.  [NSA] §04 motivates
contiguous blocks for selection (scattered reads are slow).

Readings taken where the page is silent:
  * a summary is the plain mean of `len` consecutive keys (values) taken
    every `stride` tokens; a summary is visible to row t iff its last token
    is <= t; a row that sees no summary gets a zero branch-1 output;
  * the selected branch ranks 64-token key blocks per (KV group, 64-token
    query block) by the branch-1 probability mass that falls inside each
    block: each summary's probability is split over the blocks it overlaps
    in proportion to the overlap, summed over the block's rows and the
    group's heads, and divided by (rows x heads) so scores lie in [0, 1];
    candidates are blocks j <= i, top-k, nothing forced;
  * per-token selection (the finer granularity of the original method):
    every query token ranks the blocks for its own KV group, with the same
    overlap split of its branch-1 probabilities, averaged over the group's
    heads; its candidates are blocks j <= t // sel_block; all heads of the
    group attend to that token's blocks (keys <= t);
  * the sliding branch sees keys t-W+1 .. t;
  * gates: out = sum over branches of sigmoid(z_b) * o_b (no normalisation);
  * summaries are stored in the dtype of the keys and values they summarise:
    with bf16 inputs, each float64 mean is rounded once to the nearest
    bfloat16 (ties to even) and branch 1 and the block scores use those
    stored values.
"""
from __future__ import annotations

import math

import numpy as np

from .prefill import masked_softmax_attention


def compress(x: np.ndarray, length: int, stride: int) -> np.ndarray:
    """Summaries c = 0 .. n-1: mean of x[..., c*stride : c*stride+length, :].

    n = (S - length) // stride + 1.  x [B,H,S,D] -> [B,H,n,D].
    """
    x = np.asarray(x, dtype=np.float64)
    S = x.shape[-2]
    n = (S - length) // stride + 1 if S >= length else 0
    out = np.empty(x.shape[:-2] + (n, x.shape[-1]))
    for c in range(n):
        out[..., c, :] = x[..., c * stride:c * stride + length, :].mean(axis=-2)
    return out


def round_to_bf16(x):
    """Each float64 value rounded to the nearest bfloat16 (8 significant bits,
    exponent range of float32), ties to the even neighbour; returned as
    float64.  Written from the format's definition: with |x| = m 2^e,
    0.5 <= m < 1, the representable neighbours are multiples of the quantum
    2^(e-8) (2^-133 below the normal range); magnitudes that round to 2^128
    or above overflow to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    quantum = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x[fin], -quantum)), quantum)   # rint: ties to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def stored_summaries(x, length, stride, dtype):
    """Summaries as the compressed branch stores them: the float64 means of
    `compress`, rounded once to `dtype` ("bf16"), or kept exact (None)."""
    ck = compress(x, length, stride)
    if dtype is None:
        return ck
    if dtype == "bf16":
        return round_to_bf16(ck)
    raise ValueError(f"unknown summary dtype {dtype!r}")


def summary_end(c, length, stride):
    """Position of the last token a summary covers."""
    return c * stride + length - 1


def cmp_attention(q, ck, cv, length, stride, scale, rows=None):
    """Branch 1: each row t attends to the summaries whose last token is <= t.

    q [B,Hq,S,D]; ck/cv [B,Hkv,n,D].  Returns out [B,Hq,S,D], lse [B,Hq,S]
    and the probabilities p [B,Hq,R,n] (zero where invisible) of the R
    evaluated rows.  rows: optional list of positions to evaluate (default
    all S, in order); other rows of out / lse are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv, n = ck.shape[1], ck.shape[2]
    G = Hq // Hkv
    ends = summary_end(np.arange(n), length, stride)
    rows = list(range(S)) if rows is None else list(rows)
    out = np.full((B, Hq, S, D), np.nan)
    lse = np.full((B, Hq, S), np.nan)
    probs = np.zeros((B, Hq, len(rows), n))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for ri, t in enumerate(rows):
                logits = (ck[b, g] @ q[b, h, t]) * scale
                vis = ends <= t
                if not vis.any():
                    out[b, h, t] = 0.0
                    lse[b, h, t] = -np.inf
                    continue
                m = logits[vis].max()
                p = np.where(vis, np.exp(logits - m), 0.0)
                l = p.sum()
                p = p / l
                probs[b, h, ri] = p
                out[b, h, t] = p @ cv[b, g]
                lse[b, h, t] = m + math.log(l)
    return out, lse, probs


def overlap_weights(n_cmp, length, stride, sel_block, n_blocks):
    """w[c, j] = |[c*stride, c*stride+length-1] ∩ [j*sel_block, (j+1)*sel_block-1]| / length."""
    w = np.zeros((n_cmp, n_blocks))
    for c in range(n_cmp):
        a0, a1 = c * stride, c * stride + length - 1
        for j in range(n_blocks):
            b0, b1 = j * sel_block, (j + 1) * sel_block - 1
            ov = min(a1, b1) - max(a0, b0) + 1
            if ov > 0:
                w[c, j] = ov / length
    return w


def cmp_block_scores(probs, Hkv, length, stride, sel_block, S, q_blocks=None):
    """score[b, g, i, j]: branch-1 probability mass inside key block j, summed
    over the rows of query block i and the query heads of group g, divided by
    (rows in block i) x (heads per group).

    probs from cmp_attention: [B,Hq,S,n] for all rows, or, with q_blocks, the
    rows of those query blocks in order.  Returns [B,Hkv,nB,nB] (rows of
    blocks not in q_blocks are NaN).
    """
    B, Hq, _, n = probs.shape
    G = Hq // Hkv
    nB = -(-S // sel_block)
    w = overlap_weights(n, length, stride, sel_block, nB)
    blocks = range(nB) if q_blocks is None else q_blocks
    out = np.full((B, Hkv, nB, nB), np.nan)
    for b in range(B):
        for g in range(Hkv):
            r0 = 0
            for i in blocks:
                t0, t1 = i * sel_block, min((i + 1) * sel_block, S)
                sl = slice(t0, t1) if q_blocks is None else slice(r0, r0 + t1 - t0)
                r0 += t1 - t0
                mass = np.zeros(n)
                for h in range(g * G, (g + 1) * G):
                    mass += probs[b, h, sl].sum(axis=0)
                out[b, g, i] = (mass @ w) / ((t1 - t0) * G)
    return out


def cmp_token_scores(probs, Hkv, length, stride, sel_block, S):
    """Per-token selection scores: score[b, g, t, j] is the branch-1
    probability mass of row t inside key block j (each summary split in
    proportion to its overlap with the block), averaged over the query heads
    of group g, so that each row of a token that sees a summary sums to 1.

    probs from cmp_attention [B,Hq,R,n] (R rows in the order evaluated).
    Returns [B,Hkv,R,nB].
    """
    B, Hq, R, n = probs.shape
    G = Hq // Hkv
    nB = -(-S // sel_block)
    w = overlap_weights(n, length, stride, sel_block, nB)
    out = np.zeros((B, Hkv, R, nB))
    for b in range(B):
        for g in range(Hkv):
            mass = probs[b, g * G:(g + 1) * G].sum(axis=0)   # [R, n]
            out[b, g] = (mass @ w) / G
    return out


def token_sparse_attention(q, k, v, idx, count, block, scale, rows=None):
    """Selected branch with per-token lists: row t of every query head of
    group g attends to the keys s <= t inside the blocks idx[b, g, t, :count].

    q [B,Hq,S,D]; k/v [B,Hkv,S,D]; idx [B,Hkv,S,W]; count [B,Hkv,S].  rows:
    optional positions to evaluate (others NaN).  Returns out, lse.
    """
    from .prefill import visible_keys
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    rows = range(S) if rows is None else rows
    out = np.full((B, Hq, S, D), np.nan)
    lse = np.full((B, Hq, S), np.nan)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for t in rows:
                keys = visible_keys(idx[b, g, t], int(count[b, g, t]), block, S)
                o, l = masked_softmax_attention(q[b, h, t][None, :], np.array([t]), keys,
                                                k[b, g], v[b, g], scale)
                out[b, h, t] = o[0]
                lse[b, h, t] = l[0]
    return out, lse


def window_attention(q, k, v, window, scale, rows=None):
    """Branch 3: row t attends to keys max(0, t-window+1) .. t."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    rows = range(S) if rows is None else rows
    out = np.full((B, Hq, S, D), np.nan)
    lse = np.full((B, Hq, S), np.nan)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for t in rows:
                keys = np.arange(max(0, t - window + 1), t + 1)
                o, l = masked_softmax_attention(q[b, h, t][None, :], np.array([t]), keys,
                                                k[b, g], v[b, g], scale)
                out[b, h, t] = o[0]
                lse[b, h, t] = l[0]
    return out, lse


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def combine(o_cmp, o_sel, o_win, z):
    """out[b,h,t] = sum over branches of sigmoid(z[b,t,h,branch]) * o_branch[b,h,t].

    o_* [B,Hq,S,D]; z [B,S,Hq,3] in branch order (compressed, selected, sliding).
    """
    gate = sigmoid(z).transpose(0, 2, 1, 3)  # [B,Hq,S,3]
    return (gate[..., 0:1] * np.asarray(o_cmp, dtype=np.float64)
            + gate[..., 1:2] * np.asarray(o_sel, dtype=np.float64)
            + gate[..., 2:3] * np.asarray(o_win, dtype=np.float64))


def forward(q, k, v, z, length, stride, sel_block, sel_k, window, scale, per_token=False,
            summary_dtype=None):
    """All three branches and the gated combine ([NSA] §03), in order.
    per_token: rank blocks per query token instead of per query block.
    summary_dtype: "bf16" stores the summaries rounded to bfloat16 before
    branch 1 uses them (as a bf16 pipeline does); None keeps them exact."""
    from .prefill import select_blocks, sparse_attention
    S = q.shape[2]
    ck = stored_summaries(k, length, stride, summary_dtype)
    cv = stored_summaries(v, length, stride, summary_dtype)
    o1, lse1, p1 = cmp_attention(q, ck, cv, length, stride, scale)
    if per_token:
        scores = cmp_token_scores(p1, k.shape[1], length, stride, sel_block, S)
        idx, cnt = select_blocks(scores, sel_k, 0, causal=True, row_block=sel_block)
        o2, _ = token_sparse_attention(q, k, v, idx, cnt, sel_block, scale)
    else:
        scores = cmp_block_scores(p1, k.shape[1], length, stride, sel_block, S)
        # causal candidates are blocks j <= i: no forced window (n_local = 0)
        idx, cnt = select_blocks(scores, sel_k, 0, causal=True)
        o2, _ = sparse_attention(q, k, v, idx, cnt, sel_block, scale)
    nB = scores.shape[-1]
    o3, _ = window_attention(q, k, v, window, scale)
    out = combine(o1, o2, o3, z)
    return {"ck": ck, "cv": cv, "o_cmp": o1, "lse_cmp": lse1, "scores": scores,
            "idx": idx, "count": cnt, "o_sel": o2, "o_win": o3, "out": out, "n_blocks": nB}
