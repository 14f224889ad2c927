"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the same plans, shapes and seeds).  The oracle checks
every selected index row it can afford and sampled outputs: query blocks
spread over the sequence (first, middle, last), sampled (sequence, KV head)
pairs for decode, and sampled query blocks of one KV group for the
three-branch path."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from dynamic_block_sparse_head_amd import binding as L
from dynamic_block_sparse_head_amd import configs, inputs
from dynamic_block_sparse_head_amd.pipeline import DecodePlan, NSAPlan, PrefillPlan
from oracle import decode as Od
from oracle import nsa as On
from oracle import prefill as Op

from _parity import check_bf16, check_indices, check_lse, nsa_check_summaries, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _prefill_full(c, groups, blocks):
    x = inputs.prefill_inputs(c, seed=0, device=DEV)
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, x["q"].dtype, DEV)
    plan.run(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    gs, go, gl = plan.scores.cpu().numpy(), plan.out, plan.lse
    G = c.G
    exact = []
    for g in groups:
        heads = slice(g * G, (g + 1) * G)
        q = to_np(x["q"][:, heads])
        k = to_np(x["k"][:, g:g + 1])
        v = to_np(x["v"][:, g:g + 1])
        s = Op.block_scores_pooled(q, k, c.block)                         # [1,1,nb,nb]
        fin = np.isfinite(s)
        assert (np.abs(gs[:, g:g + 1][fin] - s[fin]) <= 2.0 ** -23 * np.abs(s[fin]) + 1e-30).all()
        exact.append(check_indices(s, gi[:, g:g + 1], gc[:, g:g + 1], c.topk, c.n_local, True))
        out, lse = Op.sparse_attention(q, k, v, gi[:, g:g + 1], gc[:, g:g + 1], c.block, c.scale,
                                       q_blocks=blocks)
        rows = np.concatenate([np.arange(i * c.block, min((i + 1) * c.block, c.S)) for i in blocks])
        check_bf16(to_np(go[:, heads][:, :, rows]), out[:, :, rows], f"{c.name} g{g}")
        check_lse(to_np(gl[:, heads][:, :, rows]), lse[:, :, rows], 2e-3, f"{c.name} g{g}")
    for (b, g, t, n) in x["needles"]:
        assert n in gi[b, g, t, :gc[b, g, t]], "planted needle not selected"
    return float(np.mean(exact))


def test_prefill_16k_full_size():
    c = configs.PREFILL_16K
    exact = _prefill_full(c, groups=range(c.Hkv), blocks=[0, 23, 24, 100, 255])
    print(f"bit-exact index rows: {exact:.3f}")


def test_prefill_64k_full_size():
    c = configs.PREFILL_64K
    exact = _prefill_full(c, groups=[0, 5], blocks=[0, 39, 40, 300, 511])
    print(f"bit-exact index rows: {exact:.3f}")


def test_decode_128k_full_size():
    c = configs.DECODE_128K
    x = inputs.decode_inputs(c, seed=0, device=DEV)
    plan = DecodePlan(c.B, c.Hq, c.Hkv, c.L, c.D, c.page, c.topk, x["q"].dtype, DEV)
    plan.build_metadata(x["k"])
    plan.run(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    gs = plan.scores.cpu().numpy()
    for (b, g) in [(0, 0), (7, 3), (15, 7)]:
        heads = slice(g * c.G, (g + 1) * c.G)
        q = to_np(x["q"][b:b + 1, heads])
        k = to_np(x["k"][b:b + 1, g:g + 1])
        v = to_np(x["v"][b:b + 1, g:g + 1])
        kmin, kmax = Od.page_minmax(k, c.page)
        assert np.array_equal(to_np(plan.kmin[b:b + 1, g:g + 1]), kmin)
        assert np.array_equal(to_np(plan.kmax[b:b + 1, g:g + 1]), kmax)
        s = Od.page_scores(q, kmin, kmax)                                 # [1,1,nP]
        assert (np.abs(gs[b, g, 0] - s[0, 0]) <= 2.0 ** -23 * np.abs(s[0, 0]) + 1e-30).all()
        check_indices(s[:, :, None, :], gi[b:b + 1, g:g + 1], gc[b:b + 1, g:g + 1], c.topk, 0, False)
        out = Od.decode_attention(q, k, v, gi[b:b + 1, g:g + 1, 0], gc[b:b + 1, g:g + 1, 0],
                                  c.page, c.scale)
        check_bf16(to_np(plan.out[b:b + 1, heads]), out, f"decode b{b} g{g}")


def _nsa_sampled(c, x, plan, g, blocks, fused=None):
    """Group g of the three-branch step checked on the query blocks `blocks`
    against the oracle run from the raw inputs: the group's summaries bit
    for bit (oracle: float64 means rounded once to bf16), branch 1 on the
    oracle's summaries, block scores and selection of those blocks, the
    selected branch at the GPU's accepted lists, the sliding branch and the
    gated output.  Returns the oracle's block scores [1,1,nb,nb] (rows of
    other blocks NaN)."""
    heads = slice(g * c.G, (g + 1) * c.G)
    q = to_np(x["q"][:, heads])
    k = to_np(x["k"][:, g:g + 1])
    v = to_np(x["v"][:, g:g + 1])
    z = to_np(x["z"][:, :, heads])
    ck, cv = nsa_check_summaries(c, x, plan.ck, plan.cv, groups=slice(g, g + 1))
    rows = [t for i in blocks for t in range(i * c.sel_block, min((i + 1) * c.sel_block, c.S))]
    o1, lse1, p1 = On.cmp_attention(q, ck, cv, c.cmp_len, c.cmp_stride, c.scale, rows=rows)
    check_bf16(to_np(plan.o_cmp[:, heads][:, :, rows]), o1[:, :, rows], "o_cmp")
    check_lse(to_np(plan.lse_cmp[:, heads][:, :, rows]), lse1[:, :, rows], 2e-3, "lse_cmp")
    sc = On.cmp_block_scores(p1, 1, c.cmp_len, c.cmp_stride, c.sel_block, c.S, q_blocks=blocks)
    gsc = to_np(plan.scores[:, g:g + 1])
    gi, gc = plan.idx[:, g:g + 1].cpu().numpy(), plan.count[:, g:g + 1].cpu().numpy()
    for i in blocks:
        assert np.abs(gsc[0, 0, i, :i + 1] - sc[0, 0, i, :i + 1]).max() < 1e-6
        check_indices(sc[:, :, i:i + 1, :], gi[:, :, i:i + 1], gc[:, :, i:i + 1], c.sel_k, 0, True,
                      rows=[i])
    o2, _ = Op.sparse_attention(q, k, v, gi, gc, c.sel_block, c.scale, q_blocks=blocks)
    check_bf16(to_np(plan.o_sel[:, heads][:, :, rows]), o2[:, :, rows], "o_sel")
    o3, _ = On.window_attention(q, k, v, c.window, c.scale, rows=rows)
    ref = On.combine(o1[:, :, rows], o2[:, :, rows], o3[:, :, rows], z[:, rows])
    if not plan.fuse_combine:
        check_bf16(to_np(plan.o_win[:, heads][:, :, rows]), o3[:, :, rows], "o_win")
    check_bf16(to_np(plan.out[:, heads][:, :, rows]), ref, "nsa out")
    if fused is not None:
        check_bf16(to_np(fused[:, heads][:, :, rows]), ref, "nsa out, fused window + combine")
    return sc


def test_nsa_32k_full_size():
    c = configs.NSA_32K
    x = inputs.nsa_inputs(c, seed=0, device=DEV)
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV, fuse_combine=False)
    plan.run(x["q"], x["k"], x["v"], x["z"])
    fused = torch.empty_like(plan.out)
    L.dsa_nsa_window_combine(x["q"], x["k"], x["v"], c.window, c.scale, plan.o_cmp, plan.o_sel,
                             x["z"], fused)
    one = torch.full_like(plan.out, float("nan"))
    L.dsa_nsa_select_window_combine(x["q"], x["k"], x["v"], plan.idx, plan.count, c.sel_block,
                                    c.window, c.scale, plan.o_cmp, x["z"], one)
    torch.cuda.synchronize()
    # the one-pass selected + sliding + combine equals the two calls bit for bit
    assert torch.equal(one.view(torch.int16), fused.view(torch.int16))
    _nsa_sampled(c, x, plan, 1, [0, 1, 16, 300, 511], fused)


def _needle_gaps(c, x):
    """Oracle score margin of every planted needle at its target query block:
    its score minus the best score outside the top-k (negative when the
    needle is not in the oracle's top-k), from the raw inputs."""
    gaps = []
    for g in range(c.Hkv):
        mine = [nd for nd in x["needles"] if nd[1] == g]
        if not mine:
            continue
        targets = sorted({t for (_, _, t, _) in mine})
        q = to_np(x["q"][:, g * c.G:(g + 1) * c.G])
        ck = On.stored_summaries(to_np(x["k"][:, g:g + 1]), c.cmp_len, c.cmp_stride, "bf16")
        rows = [t for i in targets for t in range(i * c.sel_block, (i + 1) * c.sel_block)]
        _, _, p = On.cmp_attention(q, ck, ck, c.cmp_len, c.cmp_stride, c.scale, rows=rows)
        sc = On.cmp_block_scores(p, 1, c.cmp_len, c.cmp_stride, c.sel_block, c.S, q_blocks=targets)
        for (_, _, t, n) in mine:
            s = sc[0, 0, t, :t + 1]
            order = sorted(range(t + 1), key=lambda j: (-s[j], j))
            gaps.append(float(s[n] - s[order[c.sel_k]]) if n in order[:c.sel_k] else -1.0)
    return gaps


def test_nsa_32k_planted_needles():
    """The 32K three-branch workload with 4 needle blocks per KV group: the
    needle strength starts at a quarter of the keys' norm scale and doubles
    until the oracle ranks every needle in its target's top-16 with a score
    margin of at least 1e-3; the GPU must then select every needle, and its
    selection and outputs at the targets (and a few other blocks) must pass
    the usual acceptance against the oracle."""
    c = replace(configs.NSA_32K, needles=4)
    alpha = 0.25
    while True:
        x = inputs.nsa_inputs(c, seed=0, device=DEV, needle_alpha=alpha)
        gaps = _needle_gaps(c, x)
        if min(gaps) >= 1e-3:
            break
        assert alpha < 1e6, "needles never reach a 1e-3 margin"
        alpha *= 2
        del x
    print(f"needle strength {alpha}: oracle margins {min(gaps):.2e} .. {max(gaps):.2e}")
    assert len(x["needles"]) == 4 * c.Hkv
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV, fuse_branches=False)
    plan.run(x["q"], x["k"], x["v"], x["z"])
    torch.cuda.synchronize()
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    for (b, g, t, n) in x["needles"]:
        assert n in gi[b, g, t, :gc[b, g, t]], f"needle {n} not selected for block {t} of group {g}"
    for g in range(c.Hkv):
        targets = sorted({t for (_, gg, t, _) in x["needles"] if gg == g})
        _nsa_sampled(c, x, plan, g, targets + [0, 300])
