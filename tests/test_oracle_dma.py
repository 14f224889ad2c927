"""Pins of the value-driven dynamic-mask oracle ([DMA] §四-§五) against
closed forms, an independent dense formulation and planted structure."""
import math

import numpy as np
import torch
import torch.nn.functional as F

from dynamic_block_sparse_head_amd import configs, inputs
from oracle import dma as M
from oracle import prefill as P


def test_softplus_identities_and_limits():
    assert M.softplus(0.0) == math.log(2.0)
    x = np.linspace(-30, 30, 121)
    assert np.max(np.abs(M.softplus(x) - M.softplus(-x) - x)) < 1e-12      # sp(x) - sp(-x) = x
    assert M.softplus(60.0) == 60.0
    assert abs(M.softplus(-60.0) - math.exp(-60.0)) < 1e-40
    assert (np.diff(M.softplus(x)) > 0).all() and (M.softplus(x) > 0).all()


def test_dynamic_weights_closed_forms():
    rng = np.random.default_rng(0)
    v = rng.standard_normal((1, 3, 5, 4))
    delta = rng.standard_normal((3, 4))
    A = np.array([0.2, 0.0, 1.5])
    w = M.dynamic_weights(v, delta, A)
    assert np.all(w[0, 1] == 1.0)                                           # A = 0
    x = float(v[0, 2, 3] @ delta[2])
    assert abs(w[0, 2, 3] - math.exp(1.5 * math.log1p(math.exp(x)))) < 1e-12
    w0 = M.dynamic_weights(np.zeros_like(v), delta, A)                      # v = 0: 2^A
    assert np.max(np.abs(w0[0] - (2.0 ** A)[:, None])) < 1e-15
    # monotone in the projection for A > 0
    order = np.argsort(v[0, 0] @ delta[0])
    assert (np.diff(w[0, 0][order]) >= 0).all()


def test_block_weights_hand_example():
    w = np.array([1.0, 5.0, 2.0, 7.0, 0.0, 3.0, 4.0])
    assert list(M.block_weights(w, 3)) == [5.0, 7.0, 4.0]
    s = M.block_scores(w[None, None], 3)[0, 0]
    assert list(s[2]) == [5.0, 7.0, 4.0] and list(s[1][:2]) == [5.0, 7.0]
    assert np.isneginf(s[0, 1:]).all() and np.isneginf(s[1, 2])


def _sdpa_bias(q, k, v, bias, scale):
    """Dense causal attention with an additive float mask (torch CPU float64)."""
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    mask = np.where(np.tril(np.ones((S, S), bool))[None, None], 0.0, -np.inf)
    mask = mask + np.repeat(bias, G, axis=1)[:, :, None, :]
    return F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(np.repeat(k, G, 1)), torch.from_numpy(np.repeat(v, G, 1)),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy()


def _small(S=256, seed=0):
    c = configs.PREFILL_16K.with_seq(S)
    x = inputs.prefill_inputs(c, seed=seed)
    d, A = inputs.dma_params(c, seed=seed)
    f = lambda t: t.to(torch.float64).numpy()
    return c, f(x["q"]), f(x["k"]), f(x["v"]), f(d), f(A)


def test_biased_attention_all_blocks_equals_dense_with_float_mask():
    c, q, k, v, d, A = _small(320)
    res = M.dma_prefill(q, k, v, d, A, c.block, topk=c.n_blocks, n_local=1, scale=c.scale)
    ref = _sdpa_bias(q, k, v, res["weights"], c.scale)
    assert np.max(np.abs(res["out"] - ref)) < 1e-12
    assert (res["count"] == np.arange(1, c.n_blocks + 1)).all()


def test_constant_bias_changes_nothing():
    c, q, k, v, d, A = _small(256)
    s = P.block_scores_pooled(q, k, c.block)
    idx, cnt = P.select_blocks(s, 1, 1, True)
    base, lb = P.sparse_attention(q, k, v, idx, cnt, c.block, c.scale)
    out, lse = M.biased_sparse_attention(q, k, v, idx, cnt, c.block, c.scale,
                                         np.full((1, c.Hkv, c.S), 2.5))
    assert np.max(np.abs(out - base)) < 1e-13
    assert np.max(np.abs(lse - (lb + 2.5))) < 1e-12


def test_planted_heavy_block_is_kept_everywhere():
    """Values of one key block aligned with Delta make its weight the largest:
    every later query block whose window does not cover it keeps it."""
    c, q, k, v, d, A = _small(1024, seed=3)
    j = 3
    v[:, :, j * c.block:(j + 1) * c.block] += 0.5 * d[None, :, None, :] / np.linalg.norm(d, axis=1)[None, :, None, None]
    res = M.dma_prefill(q, k, v, d, A, c.block, topk=2, n_local=2, scale=c.scale)
    bw = M.block_weights(res["weights"], c.block)
    assert (bw.argmax(axis=-1) == j).all()
    for g in range(c.Hkv):
        for i in range(j + 2, c.n_blocks):
            assert j in res["idx"][0, g, i, :res["count"][0, g, i]]


def test_selection_is_top_k_of_block_weights():
    """Brute force: the kept blocks of each row are the k heaviest candidates."""
    c, q, k, v, d, A = _small(768, seed=5)
    res = M.dma_prefill(q, k, v, d, A, c.block, topk=3, n_local=1, scale=c.scale)
    bw = M.block_weights(res["weights"], c.block)
    for g in range(c.Hkv):
        for i in range(c.n_blocks):
            cands = list(range(0, i))
            top = sorted(cands, key=lambda x: (-bw[0, g, x], x))[:3]
            assert sorted(set(top) | {i}) == list(res["idx"][0, g, i, :res["count"][0, g, i]])
