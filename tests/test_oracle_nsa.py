"""Pins for the three-branch (compressed / selected / sliding) oracle.

[NSA] §03: three branches over the causal history, fused per token by
gates.  The checks: exact limits where every branch collapses to dense
causal attention, the probability-mass invariant of the block scores, and
a hand-worked block-score example (tests/golden/nsa_block_scores_example.json).
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from dynamic_block_sparse_head_amd import configs, inputs
from oracle import nsa as N
from oracle import prefill as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return t.to(torch.float64).cpu().numpy()


def _sdpa_causal(q, k, v, scale):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    return F.scaled_dot_product_attention(q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1),
                                          is_causal=True, scale=scale).numpy()


def _small(S=256, Hq=8, Hkv=2, seed=0):
    from dataclasses import replace
    c = replace(configs.NSA_32K, S=S, Hq=Hq, Hkv=Hkv)
    x = inputs.nsa_inputs(c, seed=seed)
    return c, _np(x["q"]), _np(x["k"]), _np(x["v"]), _np(x["z"])


def test_compress_identity_and_arange():
    x = np.arange(40, dtype=np.float64).reshape(1, 1, 40, 1)
    assert np.array_equal(N.compress(x, 1, 1), x)
    ck = N.compress(x, 32, 16)     # (40-32)//16 + 1 = 1 summary: tokens 0..31
    assert ck.shape[2] == 1 and ck[0, 0, 0, 0] == 15.5
    y = np.arange(64, dtype=np.float64).reshape(1, 1, 64, 1)
    ck = N.compress(y, 32, 16)     # starts 0, 16, 32 -> means 15.5, 31.5, 47.5
    assert list(ck[0, 0, :, 0]) == [15.5, 31.5, 47.5]


def test_unit_compression_is_dense_causal():
    """len = stride = 1: the summaries are the keys themselves and branch 1 is
    dense causal attention."""
    c, q, k, v, _ = _small(S=128)
    ck, cv = N.compress(k, 1, 1), N.compress(v, 1, 1)
    o1, lse, p = N.cmp_attention(q, ck, cv, 1, 1, c.scale)
    assert np.max(np.abs(o1 - _sdpa_causal(q, k, v, c.scale))) < 1e-12
    assert np.max(np.abs(p.sum(-1) - 1)) < 1e-12


def test_rows_without_a_summary_are_zero():
    c, q, k, v, _ = _small(S=128)
    ck, cv = N.compress(k, 32, 16), N.compress(v, 32, 16)
    o1, lse, p = N.cmp_attention(q, ck, cv, 32, 16, c.scale)
    assert (o1[:, :, :31] == 0).all() and np.isneginf(lse[:, :, :31]).all()
    assert np.isfinite(lse[:, :, 31:]).all()
    # row 31 sees only summary 0; row 47 sees summaries 0 and 1
    assert np.allclose(o1[:, :, 31], np.repeat(cv[:, :, 0], c.G, axis=1), atol=1e-15, rtol=0)
    assert (p[:, :, 47, 2:] == 0).all() and (p[:, :, 47, :2] > 0).all()


def test_window_limits():
    c, q, k, v, _ = _small(S=128)
    o, _ = N.window_attention(q, k, v, 1000, c.scale)
    assert np.max(np.abs(o - _sdpa_causal(q, k, v, c.scale))) < 1e-12
    o, _ = N.window_attention(q, k, v, 1, c.scale)
    assert np.max(np.abs(o - np.repeat(v, c.G, axis=1))) < 1e-15


def test_every_branch_dense_gives_closed_form():
    """len = stride = 1, k >= blocks, window >= S: each branch is dense causal
    attention, so out = (sigmoid(z1)+sigmoid(z2)+sigmoid(z3)) * dense."""
    c, q, k, v, z = _small(S=192)
    res = N.forward(q, k, v, z, 1, 1, c.sel_block, 10, 10_000, c.scale)
    dense = _sdpa_causal(q, k, v, c.scale)
    gsum = (1 / (1 + np.exp(-z))).sum(-1).transpose(0, 2, 1)[..., None]
    assert np.max(np.abs(res["out"] - gsum * dense)) < 1e-12


def test_block_scores_mass_invariant():
    """Each summary's probability is split over blocks with weights summing
    to one, so a row of block scores sums to the fraction of (row, head)
    pairs in the query block that see at least one summary."""
    c, q, k, v, _ = _small(S=256)
    ck, cv = N.compress(k, c.cmp_len, c.cmp_stride), N.compress(v, c.cmp_len, c.cmp_stride)
    _, _, p = N.cmp_attention(q, ck, cv, c.cmp_len, c.cmp_stride, c.scale)
    s = N.cmp_block_scores(p, c.Hkv, c.cmp_len, c.cmp_stride, c.sel_block, c.S)
    w = N.overlap_weights(ck.shape[2], c.cmp_len, c.cmp_stride, c.sel_block, c.n_blocks)
    assert np.allclose(w.sum(1), 1.0, atol=0, rtol=0)
    for i in range(c.n_blocks):
        t = np.arange(i * c.sel_block, (i + 1) * c.sel_block)
        frac = np.mean(t >= c.cmp_len - 1)
        assert np.allclose(s[:, :, i].sum(-1), frac, atol=1e-13)
        assert (s[:, :, i, i + 1:] == 0).all()     # no mass after the query block


def test_block_scores_hand_example():
    """Uniform logits (q = 0): scores worked out by hand in the golden file."""
    with open(os.path.join(GOLDEN, "nsa_block_scores_example.json")) as f:
        ex = json.load(f)
    S, L, st, sb = ex["S"], ex["len"], ex["stride"], ex["sel_block"]
    rng = np.random.default_rng(0)
    q = np.zeros((1, 1, S, 4))
    k = rng.standard_normal((1, 1, S, 4))
    v = rng.standard_normal((1, 1, S, 4))
    ck, cv = N.compress(k, L, st), N.compress(v, L, st)
    _, _, p = N.cmp_attention(q, ck, cv, L, st, 0.5)
    s = N.cmp_block_scores(p, 1, L, st, sb, S)
    want = np.array([[eval(x, {}) for x in row] for row in ex["scores_expr"]])
    assert np.max(np.abs(s[0, 0] - want)) < 1e-14


def test_selected_branch_uses_top16_of_candidates():
    c, q, k, v, z = _small(S=256 * 8, Hq=4, Hkv=1)
    ck, cv = N.compress(k, c.cmp_len, c.cmp_stride), N.compress(v, c.cmp_len, c.cmp_stride)
    _, _, p = N.cmp_attention(q, ck, cv, c.cmp_len, c.cmp_stride, c.scale)
    s = N.cmp_block_scores(p, c.Hkv, c.cmp_len, c.cmp_stride, c.sel_block, c.S)
    idx, cnt = P.select_blocks(s, c.sel_k, 0, causal=True)
    for i in range(c.n_blocks):
        assert cnt[0, 0, i] == min(i + 1, c.sel_k)
        chosen = set(idx[0, 0, i, :cnt[0, 0, i]])
        rest = [j for j in range(i + 1) if j not in chosen]
        if rest:
            assert min(s[0, 0, i, j] for j in chosen) >= max(s[0, 0, i, j] for j in rest)


def test_combine_gates():
    rng = np.random.default_rng(2)
    o = [rng.standard_normal((1, 2, 3, 4)) for _ in range(3)]
    z = np.zeros((1, 3, 2, 3))
    assert np.allclose(N.combine(*o, z), 0.5 * (o[0] + o[1] + o[2]), atol=1e-15, rtol=0)
    z[..., 1] = 60.0
    z[..., 0] = z[..., 2] = -60.0
    assert np.allclose(N.combine(*o, z), o[1], atol=1e-15, rtol=0)


# ----------------------------------------------------- per-token selection
def test_token_scores_hand_example():
    """Uniform logits (q = 0), two identical heads: per-row scores worked out
    by hand in the golden file; the head mean leaves them unchanged."""
    with open(os.path.join(GOLDEN, "nsa_token_scores_example.json")) as f:
        ex = json.load(f)
    S, L, st, sb = ex["S"], ex["len"], ex["stride"], ex["sel_block"]
    rng = np.random.default_rng(1)
    q = np.zeros((1, 2, S, 4))
    k = rng.standard_normal((1, 1, S, 4))
    v = rng.standard_normal((1, 1, S, 4))
    ck, cv = N.compress(k, L, st), N.compress(v, L, st)
    _, _, p = N.cmp_attention(q, ck, cv, L, st, 0.5)
    s = N.cmp_token_scores(p, 1, L, st, sb, S)
    assert s.shape == (1, 1, S, 2)
    for t0, t1, e0, e1 in ex["rows"]:
        want = np.array([eval(e0, {}), eval(e1, {})])
        assert np.max(np.abs(s[0, 0, t0:t1 + 1] - want)) < 1e-14, (t0, t1)


def test_token_scores_mass_and_block_mean():
    """A token's scores sum to 1 once it sees a summary (0 before), nothing
    falls after its own block, and the mean over a query block's rows is the
    (separately pinned) per-block score of that block."""
    c, q, k, v, _ = _small(S=320)
    ck, cv = N.compress(k, c.cmp_len, c.cmp_stride), N.compress(v, c.cmp_len, c.cmp_stride)
    _, _, p = N.cmp_attention(q, ck, cv, c.cmp_len, c.cmp_stride, c.scale)
    s = N.cmp_token_scores(p, c.Hkv, c.cmp_len, c.cmp_stride, c.sel_block, c.S)
    t = np.arange(c.S)
    want = (t >= c.cmp_len - 1).astype(np.float64)
    assert np.max(np.abs(s.sum(-1) - want)) < 1e-13
    for tt in range(c.S):
        assert (s[:, :, tt, tt // c.sel_block + 1:] == 0).all()
    sb = N.cmp_block_scores(p, c.Hkv, c.cmp_len, c.cmp_stride, c.sel_block, c.S)
    for i in range(c.n_blocks):
        rows = slice(i * c.sel_block, min((i + 1) * c.sel_block, c.S))
        assert np.max(np.abs(s[:, :, rows].mean(axis=2) - sb[:, :, i])) < 1e-14


def test_per_token_selection_brute_force():
    """Per-token candidates are blocks 0 .. t // block; against a lexsort of
    each row's candidates (ties broken by lower index), with planted ties."""
    rng = np.random.default_rng(3)
    S, blk, nK, k = 200, 16, 13, 4
    s = rng.integers(0, 5, size=(2, S, nK)).astype(np.float64)   # many ties
    idx, cnt = P.select_blocks(s, k, 0, causal=True, row_block=blk)
    for r in range(2):
        for t in range(S):
            cands = np.arange(t // blk + 1)
            order = np.lexsort((cands, -s[r, t, cands]))
            want = np.sort(cands[order[:k]])
            assert cnt[r, t] == len(want)
            assert list(idx[r, t, :cnt[r, t]]) == list(want)
            assert (idx[r, t, cnt[r, t]:] == -1).all()


def _dense_masked(q, k, v, mask, scale):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                          scale=scale).numpy()


def test_token_attention_matches_dense_masked_sdpa():
    """Every head of a group attends, per row, to the keys <= t of that
    row's own blocks: a dense SDPA with the explicit boolean mask."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, S, D, blk, kk = 1, 4, 2, 96, 8, 16, 2
    q = rng.standard_normal((B, Hq, S, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    s = rng.standard_normal((B, Hkv, S, S // blk))
    idx, cnt = P.select_blocks(s, kk, 0, causal=True, row_block=blk)
    out, lse = N.token_sparse_attention(q, k, v, idx, cnt, blk, 0.3)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        mask = np.zeros((S, S), dtype=bool)
        for t in range(S):
            for j in idx[0, g, t, :cnt[0, g, t]]:
                mask[t, j * blk:(j + 1) * blk] = True
        mask &= np.tril(np.ones((S, S), dtype=bool))
        ref = _dense_masked(q[0, h][None], k[0, g][None], v[0, g][None], mask, 0.3)[0]
        assert np.max(np.abs(out[0, h] - ref)) < 1e-12
        logits = np.where(mask, 0.3 * q[0, h] @ k[0, g].T, -np.inf)
        m = logits.max(-1)
        assert np.max(np.abs(lse[0, h] - (m + np.log(np.exp(logits - m[:, None]).sum(-1))))) < 1e-12


def test_per_token_forward_dense_limit():
    """With at least as many selected blocks as there are blocks, the
    per-token selected branch is dense causal attention."""
    c, q, k, v, z = _small(S=256, Hq=4, Hkv=1)
    res = N.forward(q, k, v, z, c.cmp_len, c.cmp_stride, c.sel_block, c.n_blocks, c.window,
                    c.scale, per_token=True)
    assert res["scores"].shape == (1, 1, c.S, c.n_blocks)
    assert np.max(np.abs(res["o_sel"] - _sdpa_causal(q, k, v, c.scale))) < 1e-12


def test_round_to_bf16_hand_cases():
    """bfloat16 keeps 8 significant bits: between 1 and 2 the spacing is
    2^-7, so 1 + 2^-8 is a tie (to the even neighbour 1), 1 + 3*2^-8 a tie
    between 1 + 2^-7 (odd last bit) and 1 + 2^-6 (even), and anything above
    a half quantum rounds up.  Below 2^-126 the spacing is 2^-133."""
    r = N.round_to_bf16
    cases = [
        (1.0, 1.0), (3.0, 3.0), (-2.5, -2.5), (0.0, 0.0),
        (1 + 2.0 ** -8, 1.0), (-(1 + 2.0 ** -8), -1.0),
        (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),
        (1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -7),
        (1 + 2.0 ** -8 - 2.0 ** -30, 1.0),
        (2.0 ** -133, 2.0 ** -133), (2.0 ** -134, 0.0), (3 * 2.0 ** -134, 2.0 ** -132),
        ((2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -7) * 2.0 ** 127),
        ((2 - 2.0 ** -8) * 2.0 ** 127, np.inf),
        (np.inf, np.inf), (-np.inf, -np.inf),
    ]
    got = r(np.array([c[0] for c in cases]))
    want = np.array([c[1] for c in cases])
    assert np.array_equal(got, want), list(zip(got, want))
    assert np.isnan(r(np.array([np.nan]))[0])


def test_round_to_bf16_matches_torch_float32_conversion():
    """For values a float32 holds exactly, rounding to bfloat16 is what
    torch's float32 -> bfloat16 conversion (round to nearest, ties to even)
    does: random bit patterns over the whole exponent range, and exact ties
    (a bfloat16 value plus half its spacing)."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    base = torch.from_numpy(rng.standard_normal(50_000).astype(np.float32)).to(torch.bfloat16)
    b64 = base.to(torch.float64).numpy()
    _, e = np.frexp(b64)
    ties = (b64 + np.ldexp(np.sign(b64), e - 9)).astype(np.float32)   # half a quantum
    for arr in (x, ties):
        want = torch.from_numpy(arr).to(torch.bfloat16).to(torch.float64).numpy()
        got = N.round_to_bf16(arr.astype(np.float64))
        same = (got == want) | (np.isnan(got) & np.isnan(want))
        assert same.all(), (arr[~same][:5], got[~same][:5], want[~same][:5])


def test_stored_summaries_of_bf16_values():
    """len = stride = 1: every summary is one bf16 key, which rounding leaves
    unchanged; len 2 of two equal keys likewise.  The stored summaries are
    the exact means rounded once."""
    c, q, k, v, _ = _small(S=96)
    assert np.array_equal(N.stored_summaries(k, 1, 1, "bf16"), k)
    kk = np.repeat(k[:, :, ::2], 2, axis=2)
    assert np.array_equal(N.stored_summaries(kk, 2, 2, "bf16"), k[:, :, ::2])
    exact = N.compress(k, 32, 16)
    stored = N.stored_summaries(k, 32, 16, "bf16")
    assert np.array_equal(stored, N.round_to_bf16(exact))
    # one rounding: within half a spacing, the unit roundoff 2^-8 relative
    assert (np.abs(stored - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-300).all()
    assert not np.array_equal(stored, exact)
