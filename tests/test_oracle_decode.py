"""Pins for the decode oracle (page selection from per-page key bounds).

[SF] §二-§四: a page-level decode method keeps the whole KV cache and reads
only selected pages.  The checks below come from the definition of the
bound (an upper bound on every q·k in the page) and from the dense limit.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from dynamic_block_sparse_head_amd import configs, inputs
from oracle import decode as Dd
from oracle import prefill as P


def _np(t):
    return t.to(torch.float64).cpu().numpy()


def _small(seed=0, L=1024, B=2):
    from dataclasses import replace
    c = replace(configs.DECODE_128K, B=B, L=L)
    x = inputs.decode_inputs(c, seed=seed)
    return c, _np(x["q"]), _np(x["k"]), _np(x["v"])


def test_minmax_bounds_and_attained():
    """kmin <= every key <= kmax, and each bound is attained by some key."""
    c, _, k, _ = _small()
    kmin, kmax = Dd.page_minmax(k, c.page)
    pages = k.reshape(c.B, c.Hkv, c.n_pages, c.page, c.D)
    assert (pages >= kmin[:, :, :, None, :]).all() and (pages <= kmax[:, :, :, None, :]).all()
    assert ((pages == kmin[:, :, :, None, :]).any(axis=3)).all()
    assert ((pages == kmax[:, :, :, None, :]).any(axis=3)).all()


def test_page_bound_is_an_upper_bound():
    """Each head's bound >= the largest q·k of any key in the page, so the
    group score >= the sum over heads of the per-head page maxima."""
    c, q, k, _ = _small()
    kmin, kmax = Dd.page_minmax(k, c.page)
    s = Dd.page_scores(q, kmin, kmax)
    for b in range(c.B):
        for g in range(c.Hkv):
            true = np.zeros(c.n_pages)
            for h in range(g * c.G, (g + 1) * c.G):
                dots = k[b, g] @ q[b, h]
                true += dots.reshape(c.n_pages, c.page).max(axis=1)
            assert (s[b, g] >= true - 1e-12).all()


def test_page_bound_equality_cases():
    """Equality when a page holds one token, or all its keys are equal; with
    q > 0 everywhere the bound is q·kmax."""
    rng = np.random.default_rng(1)
    B, Hq, Hkv, D = 1, 4, 2, 16
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, 8, D))
    kmin, kmax = Dd.page_minmax(k, 1)                       # page = 1 token
    s = Dd.page_scores(q, kmin, kmax)
    want = np.stack([sum(k[0, g] @ q[0, h] for h in range(2 * g, 2 * g + 2)) for g in range(Hkv)])
    assert np.max(np.abs(s[0] - want)) < 1e-12
    keq = np.repeat(k[:, :, :1], 8, axis=2)                 # all keys of the page equal
    kmin, kmax = Dd.page_minmax(keq, 8)
    s = Dd.page_scores(q, kmin, kmax)
    want = np.array([sum(keq[0, g, 0] @ q[0, h] for h in range(2 * g, 2 * g + 2)) for g in range(Hkv)])
    assert np.max(np.abs(s[0, :, 0] - want)) < 1e-12
    qpos = np.abs(q) + 0.1
    kmin, kmax = Dd.page_minmax(k, 4)
    s = Dd.page_scores(qpos, kmin, kmax)
    want = np.zeros_like(s)
    for g in range(Hkv):
        for h in range(2 * g, 2 * g + 2):
            want[0, g] += kmax[0, g] @ qpos[0, h]
    assert np.max(np.abs(s - want)) < 1e-12


def test_all_pages_equals_dense_single_query():
    """Selecting every page reduces to dense attention of the one query over
    the whole cache (torch CPU float64 SDPA, no mask)."""
    c, q, k, v = _small(L=512)
    kmin, kmax = Dd.page_minmax(k, c.page)
    s = Dd.page_scores(q, kmin, kmax)
    idx, cnt = P.select_blocks(s[:, :, None, :], c.n_pages, 0, causal=False)
    out = Dd.decode_attention(q, k, v, idx[:, :, 0], cnt[:, :, 0], c.page, c.scale)
    qt = torch.from_numpy(q)[:, :, None, :]
    kt = torch.from_numpy(k).repeat_interleave(c.G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(c.G, dim=1)
    ref = F.scaled_dot_product_attention(qt, kt, vt, scale=c.scale)[:, :, 0].numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_decode_selection_picks_highest_bounds():
    """Selected pages are the k largest bounds (ties: lower page), ascending."""
    c, q, k, _ = _small(L=2048)
    kmin, kmax = Dd.page_minmax(k, c.page)
    s = Dd.page_scores(q, kmin, kmax)
    kk = 5
    idx, cnt = P.select_blocks(s[:, :, None, :], kk, 0, causal=False)
    for b in range(c.B):
        for g in range(c.Hkv):
            order = sorted(range(c.n_pages), key=lambda p: (-s[b, g, p], p))[:kk]
            assert list(idx[b, g, 0]) == sorted(order)
            assert cnt[b, g, 0] == kk


def test_decode_output_is_masked_dense_over_selected_pages():
    """Same result as dense attention with -inf outside the chosen pages."""
    c, q, k, v = _small(L=1024, B=1)
    kmin, kmax = Dd.page_minmax(k, c.page)
    s = Dd.page_scores(q, kmin, kmax)
    idx, cnt = P.select_blocks(s[:, :, None, :], 3, 0, causal=False)
    out = Dd.decode_attention(q, k, v, idx[:, :, 0], cnt[:, :, 0], c.page, c.scale)
    for h in range(c.Hq):
        g = h // c.G
        allowed = np.zeros(c.L, bool)
        for p in idx[0, g, 0, :cnt[0, g, 0]]:
            allowed[p * c.page:(p + 1) * c.page] = True
        logits = (k[0, g] @ q[0, h]) * c.scale
        logits[~allowed] = -np.inf
        w = np.exp(logits - logits.max())
        w /= w.sum()
        assert np.max(np.abs(w @ v[0, g] - out[0, h])) < 1e-12
