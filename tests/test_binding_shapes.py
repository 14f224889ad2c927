"""The Python binding checks every tensor's full shape before a call goes
down to the C ABI, which only sees bare pointers: a mis-sized output or
input raises ValueError and nothing is launched.  Runs on the CPU: the
shape checks come before the device check, so correctly shaped CPU tensors
get as far as the "must be a GPU tensor" refusal and mis-sized ones stop
at their shape."""
import os

import pytest
import torch

from dynamic_block_sparse_head_amd import binding as L

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libdsa.so not built")

bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def _ok(fn, *args):
    with pytest.raises(ValueError, match="GPU tensor"):
        fn(*args)


def _bad(fn, *args, name=""):
    with pytest.raises(ValueError, match=f"{name}.*(shape|dimensions)"):
        fn(*args)


B, Hq, Hkv, S, D, blk = 1, 8, 2, 256, 128, 64
nb = S // blk


def test_prefill_shapes():
    q, k, v, out = z(B, Hq, S, D), z(B, Hkv, S, D), z(B, Hkv, S, D), z(B, Hq, S, D)
    lse = z(B, Hq, S, dtype=f32)
    idx, cnt = z(B, Hkv, nb, 3, dtype=i32), z(B, Hkv, nb, dtype=i32)
    f = L.dsa_sparse_attn_prefill
    _ok(f, q, k, v, idx, cnt, blk, 0, 0.1, out, lse)
    _bad(f, q, k, v, idx, cnt, blk, 0, 0.1, z(B, Hq, S - 1, D), lse, name="out")
    _bad(f, q, k, z(B, Hkv, S, 64), idx, cnt, blk, 0, 0.1, out, lse, name="v")
    _bad(f, q, z(B, Hkv, S + 64, D), v, idx, cnt, blk, 0, 0.1, out, lse, name="k")
    _bad(f, q, k, v, z(B, Hkv, nb - 1, 3, dtype=i32), cnt, blk, 0, 0.1, out, lse, name="idx")
    _bad(f, q, k, v, idx, z(B, Hkv, nb + 1, dtype=i32), blk, 0, 0.1, out, lse, name="count")
    _bad(f, q, k, v, idx, cnt, blk, 0, 0.1, out, z(B, Hq, S + 1, dtype=f32), name="lse")
    ex = L.dsa_sparse_attn_prefill_ex
    _ok(ex, q, k, v, z(B, Hq, nb, 3, dtype=i32), z(B, Hq, nb, dtype=i32), blk, 1,
        z(B, Hkv, S, dtype=f32), 0.1, out, lse)
    _bad(ex, q, k, v, idx, cnt, blk, 1, None, 0.1, out, lse, name="idx")   # per-head lists
    _bad(ex, q, k, v, idx, cnt, blk, 4, z(B, Hkv, S - 1, dtype=f32), 0.1, out, lse,
         name="key_bias")


def test_backward_shapes():
    q, k, v, out = z(B, Hq, S, D), z(B, Hkv, S, D), z(B, Hkv, S, D), z(B, Hq, S, D)
    lse, dout = z(B, Hq, S, dtype=f32), z(B, Hq, S, D)
    idx, cnt = z(B, Hkv, nb, 3, dtype=i32), z(B, Hkv, nb, dtype=i32)
    ws = z(1024, dtype=torch.uint8)
    dq, dk, dv = z(B, Hq, S, D), z(B, Hkv, S, D), z(B, Hkv, S, D)
    f = L.dsa_sparse_attn_prefill_backward
    _ok(f, q, k, v, out, lse, dout, idx, cnt, blk, 0.1, ws, dq, dk, dv)
    _bad(f, q, k, v, out, lse, dout, idx, cnt, blk, 0.1, ws, dq, z(B, Hq, S, D), dv, name="dk")
    _bad(f, q, k, v, out, lse, z(B, Hq, S, 64), idx, cnt, blk, 0.1, ws, dq, dk, dv, name="dout")


def test_topk_shapes():
    s = z(2, nb, nb, dtype=f32)
    f = L.dsa_topk_select
    _ok(f, s, 2, 1, True, z(2, nb, 3, dtype=i32), z(2, nb, dtype=i32))
    _bad(f, s, 2, 1, True, z(2, nb, 2, dtype=i32), z(2, nb, dtype=i32), name="idx")   # width k
    _bad(f, s, 2, 1, True, z(2, nb, 3, dtype=i32), z(2, nb - 1, dtype=i32), name="count")
    g = L.dsa_topk_select_tokens
    st = z(2, S, nb, dtype=f32)
    _ok(g, st, 2, 0, blk, z(2, S, 2, dtype=i32), z(2, S, dtype=i32))
    _bad(g, st, 2, 0, blk, z(2, S, 3, dtype=i32), z(2, S, dtype=i32), name="idx")


def test_scores_and_decode_shapes():
    q, k = z(B, Hq, S, D), z(B, Hkv, S, D)
    ws = z(1024, dtype=torch.uint8)
    f = L.dsa_block_scores
    _ok(f, L.DSA_SCORE_POOLED, q, k, None, blk, ws, z(B, Hkv, nb, nb, dtype=f32))
    _bad(f, L.DSA_SCORE_POOLED, q, k, None, blk, ws, z(B, Hq, nb, nb, dtype=f32), name="scores")
    _ok(f, L.DSA_SCORE_POOLED_HEAD, q, k, None, blk, ws, z(B, Hq, nb, nb, dtype=f32))
    Lc, page, W = 1024, 64, 4
    qd, kc, vc = z(2, Hq, D), z(2, Hkv, Lc, D), z(2, Hkv, Lc, D)
    km = z(2, Hkv, Lc // page, D)
    _ok(f, L.DSA_SCORE_PAGE_BOUND, qd, km, km, page, None, z(2, Hkv, 1, Lc // page, dtype=f32))
    _bad(f, L.DSA_SCORE_PAGE_BOUND, qd, km, z(2, Hkv, Lc // page - 1, D), page, None,
         z(2, Hkv, Lc // page, dtype=f32), name="kmax")
    _ok(L.dsa_page_minmax, kc, page, km, km)
    _bad(L.dsa_page_minmax, kc, page, z(2, Hkv, 8, D), km, name="kmin")
    idx, cnt, out = z(2, Hkv, 1, W, dtype=i32), z(2, Hkv, 1, dtype=i32), z(2, Hq, D)
    dec = L.dsa_sparse_attn_decode
    _ok(dec, qd, kc, vc, idx, cnt, page, 0.1, ws, out)
    _bad(dec, qd, kc, z(2, Hkv, Lc - 64, D), idx, cnt, page, 0.1, ws, out, name="v_cache")
    _bad(dec, qd, kc, vc, idx, z(2, Hkv + 1, dtype=i32), page, 0.1, ws, out, name="count")
    _bad(dec, qd, kc, vc, idx, cnt, page, 0.1, ws, z(2, Hq, 64), name="out")


def test_paged_shapes():
    n_pool, page, mp = 10, 64, 4
    kn, pool = z(2, Hkv, D), z(n_pool, Hkv, page, D)
    km = z(n_pool, Hkv, D)
    table, seq = z(2, mp, dtype=i32), z(2, dtype=i32)
    _ok(L.dsa_paged_append, kn, kn, table, seq, pool, pool, km, km)
    _bad(L.dsa_paged_append, kn, kn, table, z(3, dtype=i32), pool, pool, km, km, name="seq_len")
    _bad(L.dsa_paged_append, kn, kn, table, seq, pool, z(n_pool, Hkv, 32, D), km, km,
         name="v_pool")
    q = z(2, Hq, D)
    _ok(L.dsa_paged_page_scores, q, km, km, page, table, seq, z(2, Hkv, 1, mp, dtype=f32))
    _bad(L.dsa_paged_page_scores, q, km, km, page, table, seq, z(2, Hkv, mp + 1, dtype=f32),
         name="scores")
    ws = z(1024, dtype=torch.uint8)
    idx, cnt = z(2, Hkv, 1, 3, dtype=i32), z(2, Hkv, 1, dtype=i32)
    _ok(L.dsa_paged_decode, q, pool, pool, table, seq, idx, cnt, 0.1, ws, z(2, Hq, D))
    _bad(L.dsa_paged_decode, q, pool, pool, table, seq, idx, cnt, 0.1, ws, z(2, Hq + 1, D),
         name="out")


def test_three_branch_shapes():
    Gq, Sn = 16, 1100
    ln, st, sb = 32, 16, 64
    nc, nbs = (Sn - ln) // st + 1, -(-Sn // sb)
    q, k = z(1, Gq, Sn, D), z(1, 1, Sn, D)
    ck = z(1, 1, nc, D)
    _ok(L.dsa_nsa_compress, k, k, ln, st, ck, ck)
    _bad(L.dsa_nsa_compress, k, k, ln, st, z(1, 1, nc + 1, D), ck, name="ck")
    lse = z(1, Gq, Sn, dtype=f32)
    _ok(L.dsa_nsa_cmp_attn, q, ck, ck, ln, st, sb, 0.1, q, lse, z(1, 1, nbs, nbs, dtype=f32))
    _bad(L.dsa_nsa_cmp_attn, q, ck, ck, ln, st, sb, 0.1, q, lse, z(1, 1, nbs, nbs - 1, dtype=f32),
         name="block_scores")
    _ok(L.dsa_nsa_cmp_token_scores, q, ck, lse, ln, st, sb, 0.1, z(1, 1, Sn, nbs, dtype=f32))
    _bad(L.dsa_nsa_cmp_token_scores, q, ck, lse, ln, st, sb, 0.1, z(1, 1, nbs, nbs, dtype=f32),
         name="scores")
    idx, cnt = z(1, 1, Sn, 16, dtype=i32), z(1, 1, Sn, dtype=i32)
    _ok(L.dsa_sparse_attn_tokens, q, k, k, idx, cnt, sb, 0.1, q, lse)
    _bad(L.dsa_sparse_attn_tokens, q, k, k, z(1, 1, nbs, 16, dtype=i32), cnt, sb, 0.1, q, lse,
         name="idx")
    zl = z(1, Sn, Gq, 3, dtype=f32)
    _ok(L.dsa_nsa_combine, q, q, q, zl, q)
    _bad(L.dsa_nsa_combine, q, q, q, z(1, Gq, Sn, 3, dtype=f32), q, name="gate_logits")
    _ok(L.dsa_nsa_window_combine, q, k, k, 512, 0.1, q, q, zl, q)
    _bad(L.dsa_nsa_window_combine, q, k, k, 512, 0.1, q, z(1, Gq, Sn - 1, D), zl, q, name="o_sel")
    idx, cnt = z(1, 1, nbs, 16, dtype=i32), z(1, 1, nbs, dtype=i32)
    _ok(L.dsa_nsa_select_window_combine, q, k, k, idx, cnt, sb, 512, 0.1, q, zl, q)
    _bad(L.dsa_nsa_select_window_combine, q, k, k, idx, z(1, 1, nbs - 1, dtype=i32), sb, 512, 0.1,
         q, zl, q, name="count")
    _bad(L.dsa_nsa_select_window_combine, q, k, k, idx, cnt, sb, 512, 0.1, z(1, Gq, Sn, D - 1), zl,
         q, name="o_cmp")
    _bad(L.dsa_nsa_select_window_combine, q, k, k, idx, cnt, sb, 512, 0.1, q, zl,
         z(1, Gq + 1, Sn, D), name="out")


def test_dma_shapes():
    v = z(B, Hkv, S, D)
    proj, gain = z(Hkv, D, dtype=f32), z(Hkv, dtype=f32)
    w, bs = z(B, Hkv, S, dtype=f32), z(B, Hkv, nb, nb, dtype=f32)
    _ok(L.dsa_dma_weights, v, proj, gain, blk, w, bs)
    _bad(L.dsa_dma_weights, v, z(Hkv, 64, dtype=f32), gain, blk, w, bs, name="proj")
    _bad(L.dsa_dma_weights, v, proj, gain, blk, w, z(B, Hkv, nb, nb + 1, dtype=f32),
         name="block_scores")
