"""Pins of the backward oracle (oracle/backward.py) against things other than
itself: central finite differences of the forward oracle, reverse-mode
differentiation of an independent dense masked formulation (torch autograd,
float64 on the CPU), exact zeros where the mask removes a key ([DMA] §四-§五),
and two identities of softmax attention."""
import numpy as np
import pytest
import torch

from oracle import backward as Ob
from oracle import prefill as Op


def _case(seed=0, B=1, Hq=2, Hkv=1, S=40, D=4, block=8, topk=1, n_local=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D + 1))     # value width differs on purpose
    do = rng.standard_normal((B, Hq, S, D + 1))
    s = Op.block_scores_pooled(q, k, block)
    idx, cnt = Op.select_blocks(s, topk, n_local, causal=True)
    return q, k, v, do, idx, cnt, block, 1.0 / np.sqrt(D)


def _loss(q, k, v, do, idx, cnt, block, scale):
    out, _ = Op.sparse_attention(q, k, v, idx, cnt, block, scale)
    return float((out * do).sum())


def test_matches_central_differences():
    q, k, v, do, idx, cnt, block, scale = _case(S=20, block=4, topk=2)
    dq, dk, dv = Ob.sparse_attention_backward(q, k, v, idx, cnt, block, scale, do)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            old = x[pos]
            x[pos] = old + h
            lp = _loss(q, k, v, do, idx, cnt, block, scale)
            x[pos] = old - h
            lm = _loss(q, k, v, do, idx, cnt, block, scale)
            x[pos] = old
            num[pos] = (lp - lm) / (2 * h)
        assert np.abs(num - g).max() < 1e-6 * max(1.0, np.abs(g).max())


def _dense_mask(idx, cnt, block, S):
    """[B,Hkv,S,S] boolean: row t sees key s (independent of the oracle's
    gather: built from the index rows and the causal rule directly)."""
    B, Hkv, nb, _ = idx.shape
    m = np.zeros((B, Hkv, S, S), dtype=bool)
    for b in range(B):
        for g in range(Hkv):
            for i in range(nb):
                for j in idx[b, g, i, :cnt[b, g, i]]:
                    m[b, g, i * block:(i + 1) * block, j * block:(j + 1) * block] = True
    return m & np.tril(np.ones((S, S), dtype=bool))[None, None]


def test_matches_autograd_of_dense_masked_attention():
    q, k, v, do, idx, cnt, block, scale = _case(seed=1, B=2, Hq=4, Hkv=2, S=48, D=8, block=8,
                                                 topk=2, n_local=2)
    dq, dk, dv = Ob.sparse_attention_backward(q, k, v, idx, cnt, block, scale, do)
    G = q.shape[1] // k.shape[1]
    mask = torch.from_numpy(_dense_mask(idx, cnt, block, q.shape[2])).repeat_interleave(G, 1)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk, vv = tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1)
    logits = (tq @ kk.transpose(-1, -2)) * scale
    p = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=-1)
    out = p @ vv
    (out * torch.from_numpy(do)).sum().backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-12 * max(1.0, np.abs(mine).max())


def test_masked_keys_get_exactly_zero_gradient():
    """With an upstream gradient on one row only, every key that row does not
    see (unselected block, or in the future) gets exactly zero gradient."""
    q, k, v, do, idx, cnt, block, scale = _case(seed=2, S=64, block=8, topk=1, n_local=1)
    t = 45
    do1 = np.zeros_like(do)
    do1[:, :, t] = do[:, :, t]
    dq, dk, dv = Ob.sparse_attention_backward(q, k, v, idx, cnt, block, scale, do1)
    seen = _dense_mask(idx, cnt, block, q.shape[2])[0, 0, t]
    assert (~seen).sum() > 40 and seen.sum() > 8
    assert (dk[0, 0, ~seen] == 0).all() and (dv[0, 0, ~seen] == 0).all()
    assert np.abs(dk[0, 0, seen]).sum() > 0 and np.abs(dv[0, 0, seen]).sum() > 0
    assert (dq[:, :, np.arange(q.shape[2]) != t] == 0).all()


def test_softmax_identities():
    """Probabilities sum to one per row, so the value gradients of a group sum
    to the upstream gradients of its heads; and shifting every key by the same
    vector leaves the query gradient unchanged (logit shift invariance)."""
    q, k, v, do, idx, cnt, block, scale = _case(seed=3, B=1, Hq=4, Hkv=2, S=32, D=4, block=8,
                                                 topk=1, n_local=1)
    dq, dk, dv = Ob.sparse_attention_backward(q, k, v, idx, cnt, block, scale, do)
    G = 2
    for g in range(2):
        assert np.allclose(dv[0, g].sum(axis=0), do[0, g * G:(g + 1) * G].sum(axis=(0, 1)), atol=1e-12)
    shift = np.random.default_rng(9).standard_normal(k.shape[-1])
    dq2, _, _ = Ob.sparse_attention_backward(q, k + shift, v, idx, cnt, block, scale, do)
    assert np.abs(dq2 - dq).max() < 1e-12 * max(1.0, np.abs(dq).max())
