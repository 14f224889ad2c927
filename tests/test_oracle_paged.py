"""Pins of the paged-cache decode oracle against the contiguous decode
oracle, dense attention and the page min/max summaries."""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import decode as Od
from oracle import paged as Pg


def _cache(seed=0, B=3, Hkv=2, G=2, D=8, page=4, lens=(13, 8, 1)):
    rng = np.random.default_rng(seed)
    max_pages = max(-(-n // page) for n in lens) + 1
    P = B * max_pages + 3
    perm = rng.permutation(P)
    table = perm[:B * max_pages].reshape(B, max_pages)
    k_pool = rng.standard_normal((P, Hkv, page, D))
    v_pool = rng.standard_normal((P, Hkv, page, D))
    kmin = np.full((P, Hkv, D), np.nan)
    kmax = np.full((P, Hkv, D), np.nan)
    seq = np.zeros(B, dtype=np.int64)
    toks_k = rng.standard_normal((B, max(lens), Hkv, D))
    toks_v = rng.standard_normal((B, max(lens), Hkv, D))
    for t in range(max(lens)):
        live = np.array([t < n for n in lens])
        kp, vp, kn, kx, s2 = Pg.append(k_pool, v_pool, kmin, kmax, table, seq, toks_k[:, t], toks_v[:, t])
        for b in range(B):          # only sequences still growing take the token
            if live[b]:
                phys = table[b, t // page]
                k_pool[phys], v_pool[phys] = kp[phys], vp[phys]
                kmin[phys], kmax[phys] = kn[phys], kx[phys]
                seq[b] = s2[b]
    q = rng.standard_normal((B, Hkv * G, D))
    return q, k_pool, v_pool, kmin, kmax, table, seq, toks_k, toks_v, page


def test_appended_summaries_equal_page_minmax_of_the_valid_tokens():
    q, kp, vp, kn, kx, table, seq, tk, tv, page = _cache()
    for b in range(len(seq)):
        k = Pg.gather(kp, table, seq, b, page)                 # [Hkv, n, D]
        assert np.array_equal(k, tk[b, :seq[b]].transpose(1, 0, 2))
        for p in range(int(Pg.n_pages(seq[b], page))):
            rows = k[:, p * page:(p + 1) * page]
            phys = table[b, p]
            assert np.array_equal(kn[phys], rows.min(axis=1))
            assert np.array_equal(kx[phys], rows.max(axis=1))


def test_full_pages_identity_table_equals_contiguous_decode():
    rng = np.random.default_rng(1)
    B, Hkv, G, L, D, page = 2, 2, 4, 32, 8, 8
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    q = rng.standard_normal((B, Hkv * G, D))
    npg = L // page
    table = np.arange(B * npg).reshape(B, npg)
    k_pool = k.reshape(B, Hkv, npg, page, D).transpose(0, 2, 1, 3, 4).reshape(B * npg, Hkv, page, D)
    v_pool = v.reshape(B, Hkv, npg, page, D).transpose(0, 2, 1, 3, 4).reshape(B * npg, Hkv, page, D)
    kmin, kmax = Od.page_minmax(k, page)
    kmin_p = kmin.transpose(0, 2, 1, 3).reshape(B * npg, Hkv, D)
    kmax_p = kmax.transpose(0, 2, 1, 3).reshape(B * npg, Hkv, D)
    seq = np.full(B, L)
    s = Pg.page_scores(q, kmin_p, kmax_p, table, seq, page)
    assert np.max(np.abs(s - Od.page_scores(q, kmin, kmax))) < 1e-12
    idx = np.array([[[0, 2, -1], [1, 3, -1]]] * B)
    cnt = np.full((B, Hkv), 2)
    o = Pg.decode(q, k_pool, v_pool, table, seq, idx, cnt, 0.3)
    assert np.max(np.abs(o - Od.decode_attention(q, k, v, idx, cnt, page, 0.3))) < 1e-12


def test_all_pages_selected_is_dense_attention_over_the_valid_prefix():
    q, kp, vp, kn, kx, table, seq, tk, tv, page = _cache(seed=2)
    B, Hq, D = q.shape
    Hkv = kp.shape[1]
    G = Hq // Hkv
    W = table.shape[1]
    idx = np.tile(np.arange(W), (B, Hkv, 1))
    cnt = np.full((B, Hkv), W)                 # includes pages past the length
    o = Pg.decode(q, kp, vp, table, seq, idx, cnt, 0.5)
    for b in range(B):
        k = torch.from_numpy(tk[b, :seq[b]].transpose(1, 0, 2)).repeat_interleave(G, 0)
        v = torch.from_numpy(tv[b, :seq[b]].transpose(1, 0, 2)).repeat_interleave(G, 0)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[b])[:, None], k, v, scale=0.5)
        assert np.max(np.abs(o[b] - ref[:, 0].numpy())) < 1e-12


def test_scores_past_the_length_are_minus_inf_and_layout_does_not_matter():
    q, kp, vp, kn, kx, table, seq, tk, tv, page = _cache(seed=3)
    s = Pg.page_scores(q, kn, kx, table, seq, page)
    for b in range(len(seq)):
        npg = int(Pg.n_pages(seq[b], page))
        assert np.isneginf(s[b, :, npg:]).all() and np.isfinite(s[b, :, :npg]).all()
    # move every page to another pool slot: nothing observable changes
    P = kp.shape[0]
    perm = np.random.default_rng(4).permutation(P)
    inv = np.argsort(perm)
    kp2, vp2, kn2, kx2 = kp[inv], vp[inv], kn[inv], kx[inv]
    table2 = perm[table]
    assert np.array_equal(Pg.page_scores(q, kn2, kx2, table2, seq, page), s)
    idx = np.tile(np.array([0, 2]), (len(seq), kp.shape[1], 1))
    cnt = np.full((len(seq), kp.shape[1]), 2)
    assert np.array_equal(Pg.decode(q, kp2, vp2, table2, seq, idx, cnt, 0.4),
                          Pg.decode(q, kp, vp, table, seq, idx, cnt, 0.4))
