"""GPU parity of per-token NSA selection ([NSA] §03 at the method's own
granularity): per-token block scores from the compressed branch, per-token
top-k, and the selected branch in which every head of a group attends to
its token's blocks.  Calls go through the C ABI; the oracle is float64."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from dynamic_block_sparse_head_amd import binding as L
from dynamic_block_sparse_head_amd import configs, inputs
from dynamic_block_sparse_head_amd.pipeline import NSAPlan
from oracle import nsa as On
from oracle import prefill as Op

from _parity import check_bf16, check_indices, check_lse, nsa_check_summaries, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCORE_TOL = 1e-5   # per-token scores lie in [0, 1]; float32 exp2 and sums over <= 16 heads


def _sync():
    torch.cuda.synchronize()


def _branch1(c, x):
    """Compressed branch on the GPU: summaries, output, lse."""
    ck = torch.empty(c.B, c.Hkv, c.n_cmp, c.D, dtype=torch.bfloat16, device=DEV)
    cv = torch.empty_like(ck)
    L.dsa_nsa_compress(x["k"], x["v"], c.cmp_len, c.cmp_stride, ck, cv)
    o1 = torch.empty_like(x["q"])
    lse = torch.empty(c.B, c.Hq, c.S, dtype=torch.float32, device=DEV)
    L.dsa_nsa_cmp_attn(x["q"], ck, cv, c.cmp_len, c.cmp_stride, c.sel_block, c.scale, o1, lse)
    return ck, cv, lse


@pytest.mark.parametrize("S,Hq,Hkv", [(1000, 16, 2), (777, 32, 2), (600, 4, 4), (300, 24, 2)])
def test_token_scores(S, Hq, Hkv):
    """Per-token scores against the oracle's probabilities on its own
    summaries (the GPU's equal them bit for bit); ragged S, G = 8, 16, 1 and
    12 (heads padded in the tile)."""
    c = replace(configs.NSA_32K, S=S, Hq=Hq, Hkv=Hkv)
    x = inputs.nsa_inputs(c, seed=S, device=DEV)
    ck, cv, lse = _branch1(c, x)
    sc = torch.full((c.B, c.Hkv, c.S, c.n_blocks), float("nan"), device=DEV)
    L.dsa_nsa_cmp_token_scores(x["q"], ck, lse, c.cmp_len, c.cmp_stride, c.sel_block, c.scale, sc)
    _sync()
    rck, rcv = nsa_check_summaries(c, x, ck, cv)
    _, _, p = On.cmp_attention(to_np(x["q"]), rck, rcv, c.cmp_len, c.cmp_stride, c.scale)
    ref = On.cmp_token_scores(p, c.Hkv, c.cmp_len, c.cmp_stride, c.sel_block, c.S)
    g = to_np(sc)
    assert np.isfinite(g).all()
    assert np.abs(g - ref).max() < SCORE_TOL


def test_token_scores_other_geometry():
    """Summaries of 16 every 8 tokens, selection blocks of 32 (a block then
    overlaps 5 summaries) and D = 64."""
    c = replace(configs.NSA_32K, S=900, Hq=8, Hkv=1, D=64)
    x = inputs.nsa_inputs(c, seed=5, device=DEV)
    ln, st, sb = 16, 8, 32
    nc = (c.S - ln) // st + 1
    ck = torch.empty(c.B, c.Hkv, nc, c.D, dtype=torch.bfloat16, device=DEV)
    cv = torch.empty_like(ck)
    L.dsa_nsa_compress(x["k"], x["v"], ln, st, ck, cv)
    o1 = torch.empty_like(x["q"])
    lse = torch.empty(c.B, c.Hq, c.S, dtype=torch.float32, device=DEV)
    L.dsa_nsa_cmp_attn(x["q"], ck, cv, ln, st, sb, c.scale, o1, lse)
    nb = -(-c.S // sb)
    sc = torch.empty(c.B, c.Hkv, c.S, nb, device=DEV)
    L.dsa_nsa_cmp_token_scores(x["q"], ck, lse, ln, st, sb, c.scale, sc)
    _sync()
    rck = On.stored_summaries(to_np(x["k"]), ln, st, "bf16")
    rcv = On.stored_summaries(to_np(x["v"]), ln, st, "bf16")
    assert np.array_equal(to_np(ck), rck) and np.array_equal(to_np(cv), rcv)
    _, _, p = On.cmp_attention(to_np(x["q"]), rck, rcv, ln, st, c.scale)
    ref = On.cmp_token_scores(p, c.Hkv, ln, st, sb, c.S)
    assert np.abs(to_np(sc) - ref).max() < SCORE_TOL


@pytest.mark.parametrize("S,block,k,n_local", [(1000, 64, 16, 0), (4096, 64, 16, 0),
                                                (333, 32, 3, 2), (2000, 128, 5, 1)])
def test_topk_tokens_bit_exact(S, block, k, n_local):
    """Same scores in, same lists out; candidates follow each token's block."""
    rows, nk = 2, -(-S // block)
    s = inputs.random_scores(rows * S, nk, seed=S + k, ties=True).reshape(rows, S, nk)
    sg = s.to(DEV)
    idx = torch.full((rows, S, k + n_local), 7, dtype=torch.int32, device=DEV)
    cnt = torch.full((rows, S), 7, dtype=torch.int32, device=DEV)
    L.dsa_topk_select_tokens(sg, k, n_local, block, idx, cnt)
    _sync()
    ri, rc = Op.select_blocks(s.double().numpy(), k, n_local, causal=True, row_block=block)
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.array_equal(cnt.cpu().numpy(), rc)


def _lists(B, Hkv, S, block, k, seed):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((B, Hkv, S, -(-S // block)))
    return Op.select_blocks(s, k, 0, causal=True, row_block=block)


@pytest.mark.parametrize("S,Hq,Hkv,block,k", [(1000, 32, 2, 64, 16), (523, 16, 1, 64, 7),
                                               (701, 8, 2, 64, 3), (257, 12, 1, 64, 40),
                                               (130, 2, 2, 64, 1)])
def test_token_attention(S, Hq, Hkv, block, k):
    """Per-token selected branch against the oracle on the same lists: ragged
    S (a partial tile of 4 tokens, a partial last block), G = 16, 16, 4, 12,
    1, lists narrower and wider than the candidates."""
    c = replace(configs.NSA_32K, S=S, Hq=Hq, Hkv=Hkv)
    x = inputs.nsa_inputs(c, seed=S + block, device=DEV)
    idx, cnt = _lists(c.B, Hkv, S, block, k, seed=S)
    out = torch.full_like(x["q"], float("nan"))
    lse = torch.full((c.B, Hq, S), float("nan"), device=DEV)
    L.dsa_sparse_attn_tokens(x["q"], x["k"], x["v"], torch.from_numpy(idx).to(DEV),
                             torch.from_numpy(cnt).to(DEV), block, c.scale, out, lse)
    _sync()
    ro, rl = On.token_sparse_attention(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), idx, cnt,
                                       block, c.scale)
    check_bf16(to_np(out), ro, "token attention")
    check_lse(to_np(lse), rl, 2e-3, "token lse")


def test_token_attention_empty_and_single_lists():
    """Rows with an empty list give 0 and lse -inf; rows whose only block is
    their own see just the keys up to themselves."""
    c = replace(configs.NSA_32K, S=300, Hq=16, Hkv=1)
    x = inputs.nsa_inputs(c, seed=9, device=DEV)
    idx, cnt = _lists(1, 1, c.S, 64, 4, seed=3)
    cnt[0, 0, 5:300:7] = 0
    idx[0, 0, 5:300:7] = -1
    own = np.arange(c.S) % 11 == 3
    idx[0, 0, own] = -1
    idx[0, 0, own, 0] = np.arange(c.S)[own] // 64
    cnt[0, 0, own] = 1
    out = torch.full_like(x["q"], float("nan"))
    lse = torch.full((1, c.Hq, c.S), float("nan"), device=DEV)
    L.dsa_sparse_attn_tokens(x["q"], x["k"], x["v"], torch.from_numpy(idx).to(DEV),
                             torch.from_numpy(cnt).to(DEV), 64, c.scale, out, lse)
    _sync()
    ro, rl = On.token_sparse_attention(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), idx, cnt, 64,
                                       c.scale)
    empty = cnt[0, 0] == 0
    assert (to_np(out)[:, :, empty] == 0).all()
    assert np.isneginf(to_np(lse)[:, :, empty]).all()
    check_bf16(to_np(out)[:, :, ~empty], ro[:, :, ~empty], "token attention")
    check_lse(to_np(lse), rl, 2e-3, "token lse")


def test_nsa_pipeline_per_token_small():
    """The whole per-token chain against the oracle's own chain from the raw
    inputs (summaries bit for bit; selection checked as an acceptable top-k
    under the oracle's scores; the selected branch at the GPU's accepted
    lists, the oracle's own output wherever the lists agree)."""
    c = replace(configs.NSA_32K, S=2048 + 64, Hq=16, Hkv=1)
    x = inputs.nsa_inputs(c, seed=0, device=DEV)
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV, per_token=True)
    plan.run(x["q"], x["k"], x["v"], x["z"])
    _sync()
    q, k, v, z = (to_np(x[n]) for n in ("q", "k", "v", "z"))
    ref = On.forward(q, k, v, z, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k, c.window, c.scale,
                     per_token=True, summary_dtype="bf16")
    nsa_check_summaries(c, x, plan.ck, plan.cv)
    check_bf16(to_np(plan.o_cmp), ref["o_cmp"], "o_cmp")
    assert np.abs(to_np(plan.scores) - ref["scores"]).max() < SCORE_TOL
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    check_indices(ref["scores"], gi, gc, c.sel_k, 0, True, rows=[t // c.sel_block for t in range(c.S)])
    if np.array_equal(gi, ref["idx"]) and np.array_equal(gc, ref["count"]):
        o2, full = ref["o_sel"], ref["out"]
    else:
        o2, _ = On.token_sparse_attention(q, k, v, gi, gc, c.sel_block, c.scale)
        full = On.combine(ref["o_cmp"], o2, ref["o_win"], z)
    check_bf16(to_np(plan.o_sel), o2, "o_sel per token")
    check_bf16(to_np(plan.out), full, "nsa per token, end to end")


def test_nsa_per_token_32k_full_size():
    """The 32K, 64-head, 4-group workload at full size; sampled tokens of one
    group checked against the oracle (scores, lists, selected branch)."""
    c = configs.NSA_32K
    x = inputs.nsa_inputs(c, seed=0, device=DEV)
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV, per_token=True)
    plan.run(x["q"], x["k"], x["v"], x["z"])
    torch.cuda.synchronize()
    g = 2
    heads = slice(g * c.G, (g + 1) * c.G)
    q = to_np(x["q"][:, heads])
    k = to_np(x["k"][:, g:g + 1])
    v = to_np(x["v"][:, g:g + 1])
    rck, rcv = nsa_check_summaries(c, x, plan.ck, plan.cv, groups=slice(g, g + 1))
    rows = [0, 30, 31, 63, 64, 1000, 4095, 4096, 20000, 32700, 32767]
    _, _, p1 = On.cmp_attention(q, rck, rcv, c.cmp_len, c.cmp_stride, c.scale, rows=rows)
    sc = On.cmp_token_scores(p1, 1, c.cmp_len, c.cmp_stride, c.sel_block, c.S)
    gsc = to_np(plan.scores[:, g:g + 1])
    gi, gc = plan.idx[:, g:g + 1].cpu().numpy(), plan.count[:, g:g + 1].cpu().numpy()
    for r, t in enumerate(rows):
        assert np.abs(gsc[0, 0, t] - sc[0, 0, r]).max() < SCORE_TOL
        check_indices(sc[:, :, r:r + 1], gi[:, :, t:t + 1], gc[:, :, t:t + 1], c.sel_k, 0, True,
                      rows=[t // c.sel_block])
    o2, _ = On.token_sparse_attention(q, k, v, gi, gc, c.sel_block, c.scale, rows=rows)
    check_bf16(to_np(plan.o_sel[:, heads][:, :, rows]), o2[:, :, rows], "o_sel per token")
