"""Pins for the prefill oracle: each check comes from the pages or from
mathematics, not from the oracle itself.

[DMA] §五: skipping masked positions gives exactly the masked dense result;
masked positions get weight zero; top-k keeps the k highest-weight
positions after the causal mask.  [SA] "策略": block-sparse = dense inside a
block, sparse between blocks.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from dynamic_block_sparse_head_amd import configs, inputs
from oracle import prefill as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return t.to(torch.float64).cpu().numpy()


def _sdpa_causal(q, k, v, scale):
    """torch CPU float64 dense causal attention with GQA head expansion."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    return F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale).numpy()


def _small_inputs(cfg, S, seed=0):
    c = cfg.with_seq(S)
    x = inputs.prefill_inputs(c, seed=seed)
    return c, _np(x["q"]), _np(x["k"]), _np(x["v"])


# ---------------------------------------------------------------- P1 exactness
@pytest.mark.parametrize("cfg,S", [(configs.TINY_F32, 256), (configs.PREFILL_16K, 512),
                                   (configs.PREFILL_64K, 640)])
def test_all_blocks_equals_dense_causal(cfg, S):
    """k >= number of blocks: the sparse result must equal dense causal
    softmax attention ([DMA] §五: skipping is exact)."""
    c, q, k, v = _small_inputs(cfg, S)
    res = P.prefill(q, k, v, c.block, topk=c.n_blocks, n_local=c.n_local, scale=c.scale)
    ref = _sdpa_causal(q, k, v, c.scale)
    assert np.max(np.abs(res["out"] - ref)) < 1e-12
    assert (res["count"] == np.arange(1, c.n_blocks + 1)[None, None, :]).all()


def test_ragged_tail_all_blocks_equals_dense_causal():
    """A sequence that is not a whole number of blocks: the short last block
    is still exact against dense causal attention."""
    c, q, k, v = _small_inputs(configs.TINY_F32, 200)
    res = P.prefill(q, k, v, c.block, topk=100, n_local=1, scale=c.scale)
    ref = _sdpa_causal(q, k, v, c.scale)
    assert np.max(np.abs(res["out"] - ref)) < 1e-12


# ----------------------------------------------------------- P2 softmax rows
def test_softmax_rows_from_identity_values():
    """With V = identity the output rows ARE the attention probabilities:
    they are >= 0, sum to 1, and are exactly 0 off the selected mask
    ([DMA] §四: masked positions get weight zero)."""
    c, q, k, _ = _small_inputs(configs.TINY_F32, 256)
    S = c.S
    v = np.broadcast_to(np.eye(S), (c.B, c.Hkv, S, S)).copy()
    s = P.block_scores_pooled(q, k, c.block)
    idx, cnt = P.select_blocks(s, c.topk, c.n_local, causal=True)
    out, _ = P.sparse_attention(q, k, v, idx, cnt, c.block, c.scale)
    assert out.min() >= 0.0
    assert np.max(np.abs(out.sum(-1) - 1.0)) < 1e-12
    for h in range(c.Hq):
        for t in range(S):
            i = t // c.block
            allowed = np.zeros(S, bool)
            for j in idx[0, h, i, :cnt[0, h, i]]:
                allowed[j * c.block:(j + 1) * c.block] = True
            allowed[t + 1:] = False
            assert (out[0, h, t, ~allowed] == 0.0).all()
            assert (out[0, h, t, allowed] > 0.0).all()


def test_output_inside_visible_value_range():
    """A convex combination of visible values stays inside their range."""
    c, q, k, v = _small_inputs(configs.PREFILL_16K, 512)
    res = P.prefill(q, k, v, c.block, c.topk, c.n_local, c.scale)
    G = c.G
    for h in range(0, c.Hq, 5):
        g = h // G
        for t in range(0, c.S, 37):
            i = t // c.block
            keys = P.visible_keys(res["idx"][0, g, i], res["count"][0, g, i], c.block, c.S)
            keys = keys[keys <= t]
            lo, hi = v[0, g, keys].min(0), v[0, g, keys].max(0)
            o = res["out"][0, h, t]
            assert (o >= lo - 1e-12).all() and (o <= hi + 1e-12).all()


# ------------------------------------------------------- P3 brute-force top-k
def _brute_topk(row, cands, k):
    """Among all k-subsets maximising the score sum, the lexicographically
    first sorted tuple (equal scores rank the lower index first)."""
    if len(cands) <= k:
        return tuple(cands)
    best, best_sum = None, -math.inf
    for sub in itertools.combinations(cands, k):
        ssum = sum(row[j] for j in sub)
        if ssum > best_sum or (ssum == best_sum and sub < best):
            best, best_sum = sub, ssum
    return best


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("ties", [False, True])
def test_topk_brute_force(seed, ties):
    rng = np.random.default_rng(seed)
    nB = 10
    for k in range(0, 4):
        for n_local in (1, 2):
            if ties:   # exact dyadic values so equal sums are exactly equal
                s = rng.integers(0, 4, size=(nB, nB)).astype(np.float64) * 0.5
            else:
                s = rng.standard_normal((nB, nB))
            idx, cnt = P.select_blocks(s[None], k, n_local, causal=True)
            for i in range(nB):
                cands = list(range(0, i - n_local + 1))
                window = set(range(max(0, i - n_local + 1), i + 1))
                want = sorted(set(_brute_topk(s[i], cands, k)) | window)
                got = list(idx[0, i, :cnt[0, i]])
                assert got == want, (i, k, n_local)
                assert cnt[0, i] == min(i + 1, k + n_local)
                assert (idx[0, i, cnt[0, i]:] == -1).all()


def test_selected_subset_attention_equals_masked_dense():
    """Attention over the chosen blocks equals dense softmax with an explicit
    -inf mask built from the same subset (no block machinery)."""
    c, q, k, v = _small_inputs(configs.TINY_F32, 256, seed=3)
    res = P.prefill(q, k, v, c.block, c.topk, c.n_local, c.scale)
    S = c.S
    for h in range(c.Hq):
        allowed = np.zeros((S, S), bool)
        for t in range(S):
            i = t // c.block
            for j in res["idx"][0, h, i, :res["count"][0, h, i]]:
                allowed[t, j * c.block:(j + 1) * c.block] = True
        allowed &= np.tril(np.ones((S, S), bool))
        logits = (q[0, h] @ k[0, h].T) * c.scale
        logits[~allowed] = -np.inf
        m = logits.max(1, keepdims=True)
        p = np.exp(logits - m)
        p /= p.sum(1, keepdims=True)
        assert np.max(np.abs(p @ v[0, h] - res["out"][0, h])) < 1e-12


def test_nan_ranks_last_and_ties_low_index():
    s = np.array([[[0.0, np.nan, 1.0, 1.0, 0.5, 9.0]]])  # one row, 6 columns
    idx, cnt = P.select_blocks(s, 3, 0, causal=False)
    assert list(idx[0, 0]) == [2, 3, 5]
    idx, cnt = P.select_blocks(s, 5, 0, causal=False)
    assert list(idx[0, 0]) == [0, 2, 3, 4, 5]


# ----------------------------------------------------------- P4 needles
@pytest.mark.parametrize("cfg,S,seed", [(configs.TINY_F32, 256, 0), (configs.TINY_F32, 256, 1),
                                        (configs.TINY_F32, 256, 2),
                                        (configs.PREFILL_16K, 4096, 0)])
def test_planted_needles_are_selected(cfg, S, seed):
    """Keys shifted along the target block's query direction must win a top-k
    slot for that target block (the score's sign and direction)."""
    c = cfg.with_seq(S)
    x = inputs.prefill_inputs(c, seed=seed)
    assert x["needles"]
    q, k = _np(x["q"]), _np(x["k"])
    s = P.block_scores_pooled(q, k, c.block)
    idx, cnt = P.select_blocks(s, c.topk, c.n_local, causal=True)
    for (b, g, t, n) in x["needles"]:
        assert n in idx[b, g, t, :cnt[b, g, t]]
        # and by a clear margin over the best non-needle candidate
        cands = [j for j in range(t - c.n_local + 1) if j != n]
        assert s[b, g, t, n] > max(s[b, g, t, j] for j in cands)


# ------------------------------------------------------ P5 pooling
def test_pooled_score_bilinearity():
    """qbar·kbar = mean over all (query row, key row) pairs of q·k, and the
    group score is the sum of its heads' scores."""
    c, q, k, _ = _small_inputs(configs.PREFILL_16K, 256)
    s = P.block_scores_pooled(q, k, c.block)
    B = c.block
    for g in range(c.Hkv):
        for i in range(c.n_blocks):
            for j in range(i + 1):
                tot = 0.0
                for h in range(g * c.G, (g + 1) * c.G):
                    qa = q[0, h, i * B:(i + 1) * B]
                    ka = k[0, g, j * B:(j + 1) * B]
                    tot += (qa @ ka.T).sum() / (B * B)
                assert abs(s[0, g, i, j] - tot) < 1e-14
            assert np.isneginf(s[0, g, i, i + 1:]).all()


def test_pool_blocks_ragged():
    x = np.arange(10, dtype=np.float64).reshape(1, 1, 10, 1)
    pb = P.pool_blocks(x, 4)
    assert list(pb[0, 0, :, 0]) == [1.5, 5.5, 8.5]


# -------------------------------------------------------- P7 local-only limit
def test_local_only_is_block_diagonal_causal():
    """k = 0 and one local block: every block attends only to itself,
    causally — per-block dense causal attention."""
    c, q, k, v = _small_inputs(configs.PREFILL_16K, 512)
    res = P.prefill(q, k, v, c.block, topk=0, n_local=1, scale=c.scale)
    for i in range(c.n_blocks):
        sl = slice(i * c.block, (i + 1) * c.block)
        ref = _sdpa_causal(q[:, :, sl], k[:, :, sl], v[:, :, sl], c.scale)
        assert np.max(np.abs(res["out"][:, :, sl] - ref)) < 1e-12


# ---------------------------------------------------- P10 GQA reduction
def test_group_of_identical_heads_scales_score():
    """Replicating one query head G times multiplies the group score by G and
    leaves the selection unchanged; G = 1 is per-head selection."""
    c, q, k, v = _small_inputs(configs.PREFILL_16K, 1024)
    q1 = q[:, ::c.G]                       # one head per group, G = 1
    s1 = P.block_scores_pooled(q1, k, c.block)
    qrep = np.repeat(q1, c.G, axis=1)      # G identical heads
    sG = P.block_scores_pooled(qrep, k, c.block)
    fin = np.isfinite(s1)
    assert np.max(np.abs(sG[fin] - c.G * s1[fin])) < 1e-15
    i1, n1 = P.select_blocks(s1, c.topk, c.n_local, True)
    iG, nG = P.select_blocks(sG, c.topk, c.n_local, True)
    assert (i1 == iG).all() and (n1 == nG).all()


# ------------------------------------------------ P11 independence per group
def test_groups_are_independent():
    c, q, k, v = _small_inputs(configs.PREFILL_16K, 512)
    base = P.prefill(q, k, v, c.block, c.topk, c.n_local, c.scale)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    g = 3
    rng = np.random.default_rng(9)
    k2[:, g] += rng.standard_normal(k2[:, g].shape)
    v2[:, g] += 1.0
    q2[:, g * c.G:(g + 1) * c.G] *= -1
    pert = P.prefill(q2, k2, v2, c.block, c.topk, c.n_local, c.scale)
    others = [x for x in range(c.Hkv) if x != g]
    heads = [h for h in range(c.Hq) if h // c.G != g]
    assert np.array_equal(base["scores"][:, others], pert["scores"][:, others])
    assert np.array_equal(base["idx"][:, others], pert["idx"][:, others])
    assert np.array_equal(base["out"][:, heads], pert["out"][:, heads])


# ------------------------------------------------ golden: a worked example
def test_hand_worked_example():
    """tests/golden/prefill_worked_example.json: selection and outputs worked
    out by hand (its "derivation" field) for a 4-block toy problem."""
    with open(os.path.join(GOLDEN, "prefill_worked_example.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"], dtype=np.float64)[None, None]
    k = np.array(ex["k"], dtype=np.float64)[None, None]
    v = np.array(ex["v"], dtype=np.float64)[None, None]
    res = P.prefill(q, k, v, ex["block"], ex["topk"], ex["n_local"], ex["scale"])
    want_s = np.array([[-np.inf if x is None else x for x in row] for row in ex["scores"]])
    assert np.array_equal(res["scores"][0, 0], want_s)
    assert res["idx"][0, 0].tolist() == ex["idx"]
    assert res["count"][0, 0].tolist() == ex["count"]
    assert np.max(np.abs(res["out"][0, 0] - np.array(ex["out"]))) < 1e-12


def test_worked_example_numbers_match_their_closed_forms():
    with open(os.path.join(GOLDEN, "prefill_worked_example.json")) as f:
        ex = json.load(f)
    for expr, row in zip(ex["out_expr"], ex["out"]):
        assert abs(eval(expr, {"e": math.e}) - row[0]) < 1e-15 and row[1] == 1.0


# --------------------------------------- per-query-head selection (sel_heads)
def test_per_head_scores_are_pairwise_means_and_sum_to_group_score():
    """sel_heads = 1: each head's score is the mean of its own q·k pairs of
    the two blocks; summing the heads of a group gives the group score."""
    c, q, k, _ = _small_inputs(configs.PREFILL_16K, 256)
    sh = P.block_scores_pooled(q, k, c.block, sel_heads=1)
    assert sh.shape == (1, c.Hq, c.n_blocks, c.n_blocks)
    B = c.block
    for h in (0, 5, c.Hq - 1):
        g = h // c.G
        for i in range(c.n_blocks):
            for j in range(i + 1):
                qa = q[0, h, i * B:(i + 1) * B]
                ka = k[0, g, j * B:(j + 1) * B]
                assert abs(sh[0, h, i, j] - (qa @ ka.T).sum() / (B * B)) < 1e-14
    sg = P.block_scores_pooled(q, k, c.block)
    fin = np.isfinite(sg)
    summed = sh.reshape(1, c.Hkv, c.G, c.n_blocks, c.n_blocks).sum(axis=2)
    assert np.max(np.abs(summed[fin] - sg[fin])) < 1e-14
    two = P.block_scores_pooled(q, k, c.block, sel_heads=2)    # pairs of heads
    assert np.max(np.abs(two[np.isfinite(two)] -
                         sh.reshape(1, c.Hq // 2, 2, c.n_blocks, c.n_blocks).sum(axis=2)[np.isfinite(two)])) < 1e-14


def test_per_head_selection_attention_equals_masked_dense():
    """sel_heads = 1 under GQA: each query head attends over its own chosen
    blocks — the same as dense softmax with that head's explicit -inf mask,
    built here from a brute-force top-k over the head's own scores."""
    c, q, k, v = _small_inputs(configs.PREFILL_16K, 384, seed=4)
    topk, n_local = 2, 1
    res = P.prefill(q, k, v, c.block, topk, n_local, c.scale, sel_heads=1)
    S, nb = c.S, c.n_blocks
    differs = False
    for h in range(c.Hq):
        g = h // c.G
        allowed = np.zeros((S, S), bool)
        for i in range(nb):
            cands = list(range(0, i - n_local + 1))
            sc = [float((q[0, h, i * c.block:(i + 1) * c.block].mean(0)) @
                        (k[0, g, j * c.block:(j + 1) * c.block].mean(0))) for j in cands]
            best = set()
            if cands:
                best = set(max(itertools.combinations(range(len(cands)), min(topk, len(cands))),
                               key=lambda cmb: (sum(sc[x] for x in cmb), [-x for x in cmb])))
                best = {cands[x] for x in best}
            chosen = sorted(best | set(range(max(0, i - n_local + 1), i + 1)))
            assert list(res["idx"][0, h, i, :res["count"][0, h, i]]) == chosen
            for j in chosen:
                allowed[i * c.block:(i + 1) * c.block, j * c.block:(j + 1) * c.block] = True
        allowed &= np.tril(np.ones((S, S), bool))
        logits = (q[0, h] @ k[0, g].T) * c.scale
        logits[~allowed] = -np.inf
        p = np.exp(logits - logits.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        assert np.max(np.abs(p @ v[0, g] - res["out"][0, h])) < 1e-12
        if h % c.G and not np.array_equal(res["idx"][0, h], res["idx"][0, h - 1]):
            differs = True
    assert differs      # the heads of a group really chose differently somewhere


def test_per_head_selection_of_identical_heads_is_the_group_selection():
    """Heads of a group that are identical rank blocks identically, so the
    per-head lists and outputs equal the per-group ones."""
    c, q, k, v = _small_inputs(configs.PREFILL_16K, 512)
    qrep = np.repeat(q[:, ::c.G], c.G, axis=1)
    grp = P.prefill(qrep, k, v, c.block, c.topk, c.n_local, c.scale)
    per = P.prefill(qrep, k, v, c.block, c.topk, c.n_local, c.scale, sel_heads=1)
    for h in range(c.Hq):
        assert np.array_equal(per["idx"][0, h], grp["idx"][0, h // c.G])
    assert np.max(np.abs(per["out"] - grp["out"])) == 0.0


def test_per_head_all_blocks_equals_dense_causal():
    c, q, k, v = _small_inputs(configs.PREFILL_16K, 320)
    res = P.prefill(q, k, v, c.block, topk=c.n_blocks, n_local=1, scale=c.scale, sel_heads=1)
    assert np.max(np.abs(res["out"] - _sdpa_causal(q, k, v, c.scale))) < 1e-12
