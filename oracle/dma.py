"""Oracle: value-driven dynamic mask — TEST INFRASTRUCTURE.

Follows [DMA] §四-§五: a per-position importance weight comes from the
value content alone, delta = exp(tau(v Delta) x A), with Delta a learned
sampling projection, A a per-head gate and tau a non-negative activation;
combined with the causal mask, the k highest-weight history positions are
kept and every other position's mask value is -inf; attention then runs over
the kept positions only.  Readings taken where the page is silent:
  * per KV head g: Delta_g in R^D projects a value row to a scalar and A_g
    is a positive scalar gain; tau = softplus(x) = log(1 + e^x);
    delta[b,g,s] = exp(A_g * softplus(v[b,g,s] . Delta_g)), independent of
    the query;
  * selection is block-granular like the rest of the library: key block j
    weighs max over its positions of delta; each query block keeps the k
    heaviest blocks among those before its local window (ties: lower index)
    plus the window;
  * a kept position's mask value is its weight: the logit of key s for a
    query row t >= s is scale * q_t . k_s + delta_s; all other keys are -inf.
Everything is float64.  Pinned in tests/test_oracle_dma.py.
"""
from __future__ import annotations

import math

import numpy as np

from .prefill import select_blocks, visible_keys


def softplus(x):
    """log(1 + e^x), evaluated without overflow."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def dynamic_weights(v, delta, A):
    """delta [B,Hkv,S] from values v [B,Hkv,S,D], projections delta_proj
    [Hkv,D] (here `delta`) and gains A [Hkv]."""
    v = np.asarray(v, dtype=np.float64)
    proj = np.einsum("bgsd,gd->bgs", v, np.asarray(delta, dtype=np.float64))
    return np.exp(np.asarray(A, dtype=np.float64)[None, :, None] * softplus(proj))


def block_weights(w, block):
    """Largest weight of each run of `block` positions along the last axis
    (the last run may be short): [..., S] -> [..., ceil(S/block)]."""
    S = w.shape[-1]
    n = -(-S // block)
    return np.stack([w[..., j * block:min((j + 1) * block, S)].max(axis=-1) for j in range(n)],
                    axis=-1)


def block_scores(w, block):
    """Selection scores [B,Hkv,nb,nb]: row i holds the key-block weights for
    j <= i (the causal part) and -inf above the diagonal."""
    bw = block_weights(w, block)
    n = bw.shape[-1]
    s = np.broadcast_to(bw[..., None, :], bw.shape[:-1] + (n, n)).copy()
    s[..., np.triu_indices(n, 1)[0], np.triu_indices(n, 1)[1]] = -np.inf
    return s


def biased_sparse_attention(q, k, v, idx, count, block, scale, bias):
    """sparse_attention with an additive per-key term: row t of query block i
    attends to keys s <= t of its selected blocks with logits
    scale * q_t . k_s + bias[b,g,s].  Returns out [B,Hq,S,D], lse [B,Hq,S]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    n = -(-S // block)
    out = np.zeros((B, Hq, S, v.shape[-1]))
    lse = np.full((B, Hq, S), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(n):
                t = np.arange(i * block, min((i + 1) * block, S))
                keys = visible_keys(idx[b, g, i], int(count[b, g, i]), block, S)
                if keys.size == 0:
                    continue
                logits = (q[b, h, t] @ k[b, g, keys].T) * scale + bias[b, g, keys][None, :]
                logits = np.where(keys[None, :] <= t[:, None], logits, -np.inf)
                for r in range(t.size):
                    row = logits[r]
                    if not np.isfinite(row).any():
                        continue
                    m = row.max()
                    p = np.exp(row - m)
                    out[b, h, t[r]] = (p @ v[b, g, keys]) / p.sum()
                    lse[b, h, t[r]] = m + math.log(p.sum())
    return out, lse


def dma_prefill(q, k, v, delta, A, block, topk, n_local, scale):
    """The whole path: weights -> block scores -> top-k + window -> biased
    sparse attention."""
    w = dynamic_weights(v, delta, A)
    s = block_scores(w, block)
    idx, cnt = select_blocks(s, topk, n_local, causal=True)
    out, lse = biased_sparse_attention(q, k, v, idx, cnt, block, scale, w)
    return {"weights": w, "scores": s, "idx": idx, "count": cnt, "out": out, "lse": lse}
