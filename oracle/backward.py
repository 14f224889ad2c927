"""Oracle: gradients of block-sparse causal attention — TEST INFRASTRUCTURE.

Follows [DMA] §四 and §五: the sparse computation stays fully
differentiable; positions the mask removes get exactly zero gradient and the
kept positions receive the ordinary softmax-attention gradient, so the
sparse backward equals the dense masked backward.  Reading taken where the
pages are silent: the selected index lists are constants of the backward
(a top-k of block scores is piecewise constant, so no gradient flows into
the scores); gradients are taken of the attention output with respect to
q, k and v.

For one query row t with visible keys V_t, logits l_s = scale q_t.k_s,
probabilities P = softmax(l) over V_t and output o_t = sum P_s v_s, an upstream
gradient do_t gives
    dP_s  = do_t . v_s
    D_t   = sum_s P_s dP_s  (= do_t . o_t)
    dl_s  = P_s (dP_s - D_t)
    dq_t  = scale sum_s dl_s k_s,  dk_s += scale dl_s q_t,  dv_s += P_s do_t.
Everything is float64; pinned in tests/test_oracle_backward.py against
central finite differences of the forward oracle and against reverse-mode
differentiation of an independent dense masked formulation.
"""
from __future__ import annotations

import numpy as np

from .prefill import visible_keys


def masked_softmax_attention_grad(q_rows, t_rows, keys, k, v, scale, dout_rows):
    """Gradients of masked_softmax_attention for rows at positions t_rows over
    key positions `keys` (each row sees keys s <= t).

    Returns (dq [R,D], dk [len(keys),D], dv [len(keys),Dv]); rows that see no
    key contribute nothing."""
    R, D = q_rows.shape
    n = keys.size
    dq = np.zeros((R, D))
    dk = np.zeros((n, D))
    dv = np.zeros((n, v.shape[-1]))
    if n == 0:
        return dq, dk, dv
    kk, vv = k[keys], v[keys]
    logits = (q_rows @ kk.T) * scale
    visible = keys[None, :] <= t_rows[:, None]
    logits = np.where(visible, logits, -np.inf)
    P = np.zeros((R, n))
    for r in range(R):
        if visible[r].any():
            e = np.exp(logits[r] - logits[r].max())
            P[r] = e / e.sum()
    dP = dout_rows @ vv.T
    Dt = (P * dP).sum(axis=1)
    dl = P * (dP - Dt[:, None])
    dq = scale * (dl @ kk)
    dk = scale * (dl.T @ q_rows)
    dv = P.T @ dout_rows
    return dq, dk, dv


def sparse_attention_backward(q, k, v, idx, count, block, scale, dout):
    """Gradients of sparse_attention (same index convention) for the upstream
    gradient dout [B,Hq,S,Dv].  Returns dq [B,Hq,S,D], dk [B,Hkv,S,D],
    dv [B,Hkv,S,Dv] (float64); a key's gradient sums over every query head of
    its group and every row that sees it."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    n = -(-S // block)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(n):
                t = np.arange(i * block, min((i + 1) * block, S))
                keys = visible_keys(idx[b, g, i], int(count[b, g, i]), block, S)
                gq, gk, gv = masked_softmax_attention_grad(q[b, h, t], t, keys, k[b, g], v[b, g],
                                                           scale, dout[b, h, t])
                dq[b, h, t] += gq
                np.add.at(dk[b, g], keys, gk)
                np.add.at(dv[b, g], keys, gv)
    return dq, dk, dv
