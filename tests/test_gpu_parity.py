"""GPU parity: every entry point of libdsa.so against the float64 oracle on
the same seeded inputs, at sizes the oracle finishes in seconds (several
tiles, ragged tails, degenerate cases).  Calls go through the C ABI."""
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

from _parity import (check_bf16, check_f32, check_index_row, check_indices, check_lse,
                     nsa_check_summaries, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------- selection
@pytest.mark.parametrize("n_q,n_k,k,n_local,causal", [
    (8, 8, 2, 1, True), (256, 256, 16, 8, True), (512, 512, 32, 8, True), (512, 512, 16, 0, True),
    (1, 2048, 102, 0, False), (1, 300, 7, 3, False), (40, 40, 0, 2, True), (33, 33, 100, 1, True),
    (64, 64, 5, 2, True), (65, 65, 5, 2, True), (2, 1024, 51, 1, False), (2, 2049, 102, 0, False),
    (1, 8192, 409, 4, False), (512, 2048, 64, 4, False), (300, 1000, 40, 2, True)])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_bit_exact(n_q, n_k, k, n_local, causal, ties):
    """Same float32 scores in, same indices out: selection is bit-exact."""
    rows = 3
    s = inputs.random_scores(rows * n_q, n_k, seed=n_k + k, ties=ties).reshape(rows, n_q, n_k)
    if causal:   # entries above the diagonal are -inf as the scorer writes them
        s = s.masked_fill(torch.triu(torch.ones(n_q, n_k, dtype=torch.bool), diagonal=1), float("-inf"))
    sg = s.to(DEV)
    idx = torch.full((rows, n_q, k + n_local), 77, dtype=torch.int32, device=DEV)
    cnt = torch.full((rows, n_q), 77, dtype=torch.int32, device=DEV)
    L.dsa_topk_select(sg, k, n_local, causal, idx, cnt)
    _sync()
    oi, oc = Op.select_blocks(s.double().numpy(), k, n_local, causal)
    assert np.array_equal(idx.cpu().numpy(), oi)
    assert np.array_equal(cnt.cpu().numpy(), oc)


def test_topk_nan_ranks_last():
    s = torch.tensor([[[0.0, float("nan"), 1.0, 1.0, 0.5, 9.0]]])
    idx = torch.empty((1, 1, 3), dtype=torch.int32, device=DEV)
    cnt = torch.empty((1, 1), dtype=torch.int32, device=DEV)
    L.dsa_topk_select(s.to(DEV), 3, 0, False, idx, cnt)
    _sync()
    assert idx.cpu().tolist() == [[[2, 3, 5]]] and cnt.item() == 3


# ---------------------------------------------------------- pooled scores
@pytest.mark.parametrize("cfg,S", [(configs.TINY_F32, 256), (configs.TINY_F32, 200),
                                   (configs.PREFILL_16K, 2048), (configs.PREFILL_64K, 2048 + 64)])
def test_pooled_scores(cfg, S):
    c = cfg.with_seq(S)
    x = inputs.prefill_inputs(c, seed=1, device=DEV)
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, x["q"].dtype, DEV)
    plan.score(x["q"], x["k"])
    _sync()
    ref = Op.block_scores_pooled(to_np(x["q"]), to_np(x["k"]), c.block)
    got = to_np(plan.scores)
    assert (np.isneginf(got) == np.isneginf(ref)).all()
    fin = np.isfinite(ref)
    # float64 accumulation rounded once to float32
    assert (np.abs(got[fin] - ref[fin]) <= 2.0 ** -23 * np.abs(ref[fin]) + 1e-30).all()


# -------------------------------------------------------------- prefill
def _prefill_parity(c, seed=0):
    x = inputs.prefill_inputs(c, seed=seed, device=DEV)
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, x["q"].dtype, DEV)
    plan.run(x["q"], x["k"], x["v"])
    _sync()
    q, k, v = to_np(x["q"]), to_np(x["k"]), to_np(x["v"])
    s_ref = Op.block_scores_pooled(q, k, c.block)
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    exact = check_indices(s_ref, gi, gc, c.topk, c.n_local, True)
    for (b, g, t, n) in x["needles"]:
        assert n in gi[b, g, t, :gc[b, g, t]], "planted needle not selected"
    out, lse = Op.sparse_attention(q, k, v, gi, gc, c.block, c.scale)
    go, gl = to_np(plan.out), to_np(plan.lse)
    if c.dtype == "f32":
        check_f32(go, out, c.name)
        check_lse(gl, lse, 1e-4, c.name)
    else:
        check_bf16(go, out, c.name)
        check_lse(gl, lse, 2e-3, c.name)
    return exact


def test_prefill_tiny_f32_full_config():
    exact = _prefill_parity(configs.TINY_F32)
    assert exact == 1.0


@pytest.mark.parametrize("seed", [1, 2])
def test_prefill_tiny_f32_seeds(seed):
    _prefill_parity(configs.TINY_F32, seed=seed)


@pytest.mark.parametrize("S", [2048, 2000])
def test_prefill_bf16_16k_shape(S):
    _prefill_parity(configs.PREFILL_16K.with_seq(S))


def test_prefill_bf16_64k_shape_mixture():
    _prefill_parity(configs.PREFILL_64K.with_seq(6144))


def test_prefill_bf16_block32_and_d64():
    c = replace(configs.PREFILL_16K, name="b32d64", S=1024 + 32, D=64, block=32, topk=5, window=64,
                q_std=0.125, kv_std=0.125, v_std=0.125, needles=2, needle_alpha=0.5)
    _prefill_parity(c)


@pytest.mark.parametrize("which", ["bf16", "f32", "b32d64"])
def test_prefill_batch_of_two(which):
    """Two sequences in one call (every kernel indexes by sequence): the 16K
    shape with a ragged tail, the float32 workload and the D = 64 / 32-token
    generic kernel."""
    if which == "bf16":
        c = replace(configs.PREFILL_16K.with_seq(1000), B=2)
    elif which == "f32":
        c = replace(configs.TINY_F32, B=2)
    else:
        c = replace(configs.PREFILL_16K, name="b32d64", B=2, S=700, D=64, block=32, topk=5,
                    window=64, q_std=0.125, kv_std=0.125, v_std=0.125, needles=2,
                    needle_alpha=0.5)
    _prefill_parity(c, seed=3)


def _nsa_end_to_end(c, x, plan, fused=None):
    """The GPU's three-branch step against the oracle's own chain from the
    raw q, k, v, z (no GPU intermediate enters the oracle): summaries bit for
    bit, branch 1 and its log-sum-exp, block scores, selection as an
    acceptable top-k under the oracle's scores, the selected branch at the
    GPU's accepted lists (the oracle's own output wherever the lists agree),
    the sliding branch and the gated output."""
    q, k, v, z = (to_np(x[n]) for n in ("q", "k", "v", "z"))
    ref = On.forward(q, k, v, z, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k, c.window, c.scale,
                     summary_dtype="bf16")
    nsa_check_summaries(c, x, plan.ck, plan.cv)
    check_bf16(to_np(plan.o_cmp), ref["o_cmp"], "o_cmp")
    check_lse(to_np(plan.lse_cmp), ref["lse_cmp"], 2e-3, "lse_cmp")
    assert np.abs(to_np(plan.scores) - ref["scores"]).max() < 1e-6
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    exact = check_indices(ref["scores"], gi, gc, c.sel_k, 0, True)
    if np.array_equal(gi, ref["idx"]) and np.array_equal(gc, ref["count"]):
        o2 = ref["o_sel"]
        full = ref["out"]
    else:   # accepted near-ties: the oracle's selected branch at the GPU's lists
        o2, _ = Op.sparse_attention(q, k, v, gi, gc, c.sel_block, c.scale)
        full = On.combine(ref["o_cmp"], o2, ref["o_win"], z)
    check_bf16(to_np(plan.o_sel), o2, "o_sel")
    if not plan.fuse_combine:
        check_bf16(to_np(plan.o_win), ref["o_win"], "o_win")
    check_bf16(to_np(plan.out), full, "nsa out, end to end")
    if fused is not None:
        check_bf16(to_np(fused), full, "nsa out with the fused window + combine, end to end")
    return exact


def test_nsa_pipeline_batch_of_two():
    """The three-branch step on two sequences, fused and two-call combines,
    end to end against the oracle."""
    c = replace(configs.NSA_32K, B=2, S=1100, Hq=8, Hkv=2)
    x = inputs.nsa_inputs(c, seed=4, device=DEV)
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV, fuse_combine=False)
    plan.run(x["q"], x["k"], x["v"], x["z"])
    fused = torch.empty_like(plan.out)
    L.dsa_nsa_window_combine(x["q"], x["k"], x["v"], c.window, c.scale, plan.o_cmp, plan.o_sel,
                             x["z"], fused)
    _sync()
    _nsa_end_to_end(c, x, plan, fused)


@pytest.mark.parametrize("S", [1, 37, 64, 65])
@pytest.mark.parametrize("which", ["bf16", "f32"])
def test_prefill_short_sequences(S, which):
    """Degenerate lengths: one token, less than one block, exactly one block,
    one block and a single-token tail."""
    base = configs.PREFILL_16K if which == "bf16" else configs.TINY_F32
    _prefill_parity(replace(base.with_seq(S), needles=0), seed=S)


def test_prefill_all_blocks_equals_dense():
    """k >= number of blocks: the kernel reproduces dense causal attention."""
    c = configs.PREFILL_16K.with_seq(1024)
    x = inputs.prefill_inputs(c, seed=3, device=DEV)
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.n_blocks, 1, x["q"].dtype, DEV)
    plan.run(x["q"], x["k"], x["v"])
    _sync()
    assert (plan.count.cpu().numpy() == np.arange(1, c.n_blocks + 1)).all()
    q, k, v = to_np(x["q"]), to_np(x["k"]), to_np(x["v"])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k).repeat_interleave(c.G, 1),
        torch.from_numpy(v).repeat_interleave(c.G, 1), is_causal=True, scale=c.scale).numpy()
    check_bf16(to_np(plan.out), ref, "dense")


def test_prefill_window_mode():
    c = replace(configs.NSA_32K, S=1000, Hq=8, Hkv=2)
    x = inputs.nsa_inputs(c, seed=0, device=DEV)
    out = torch.empty_like(x["q"])
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device=DEV)
    for W in (512, 100, 1):
        L.dsa_sparse_attn_prefill(x["q"], x["k"], x["v"], None, None, 64, W, c.scale, out, lse)
        _sync()
        ref, rl = On.window_attention(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), W, c.scale)
        check_bf16(to_np(out), ref, f"window {W}")
        check_lse(to_np(lse), rl, 2e-3, f"window {W}")


def test_prefill_deterministic():
    c = configs.PREFILL_16K.with_seq(2048)
    x = inputs.prefill_inputs(c, seed=5, device=DEV)
    p = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, x["q"].dtype, DEV)
    p.run(x["q"], x["k"], x["v"])
    a = (p.scores.clone(), p.idx.clone(), p.out.clone(), p.lse.clone())
    p.run(x["q"], x["k"], x["v"])
    _sync()
    for u, w in zip(a, (p.scores, p.idx, p.out, p.lse)):
        assert torch.equal(u, w)


# --------------------------------------------------------------- decode
def _decode_parity(B=2, L_=8192, topk=6, seed=0, page=64, Hq=32, Hkv=8):
    c = replace(configs.DECODE_128K, B=B, L=L_, page=page, Hq=Hq, Hkv=Hkv)
    x = inputs.decode_inputs(c, seed=seed, device=DEV)
    plan = DecodePlan(c.B, c.Hq, c.Hkv, c.L, c.D, c.page, topk, x["q"].dtype, DEV)
    plan.build_metadata(x["k"])
    plan.run(x["q"], x["k"], x["v"])
    _sync()
    q, k, v = to_np(x["q"]), to_np(x["k"]), to_np(x["v"])
    kmin, kmax = Od.page_minmax(k, c.page)
    assert np.array_equal(to_np(plan.kmin), kmin) and np.array_equal(to_np(plan.kmax), kmax)
    s = Od.page_scores(q, kmin, kmax)
    got = to_np(plan.scores)[:, :, 0]
    assert (np.abs(got - s) <= 2.0 ** -23 * np.abs(s) + 1e-30).all()
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    check_indices(s[:, :, None, :], gi, gc, topk, 0, False)
    ref = Od.decode_attention(q, k, v, gi[:, :, 0], gc[:, :, 0], c.page, c.scale)
    check_bf16(to_np(plan.out), ref, "decode")


def test_decode_small():
    _decode_parity()


def test_decode_odd_counts_and_page128():
    _decode_parity(B=1, L_=128 * 40, topk=13, page=128, seed=2)


@pytest.mark.parametrize("page,Hq", [(32, 32), (256, 32), (64, 16), (64, 64)])
def test_decode_page_sizes_and_group_sizes(page, Hq):
    """Four heads per KV head with 32- and 256-token pages (the per-row pair
    reduction with two pages per slab and four slabs per page), and two and
    eight heads per KV head (the per-lane reduction)."""
    _decode_parity(B=2, L_=page * 48, topk=7, page=page, Hq=Hq, Hkv=8, seed=page + Hq)


def test_decode_all_pages_is_dense():
    c = replace(configs.DECODE_128K, B=1, L=2048)
    x = inputs.decode_inputs(c, seed=4, device=DEV)
    plan = DecodePlan(c.B, c.Hq, c.Hkv, c.L, c.D, c.page, c.L // c.page, x["q"].dtype, DEV)
    plan.build_metadata(x["k"])
    plan.run(x["q"], x["k"], x["v"])
    _sync()
    q, k, v = (torch.from_numpy(to_np(x[n])) for n in ("q", "k", "v"))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[:, :, None], k.repeat_interleave(c.G, 1), v.repeat_interleave(c.G, 1), scale=c.scale)[:, :, 0]
    check_bf16(to_np(plan.out), ref.numpy(), "dense decode")


# ------------------------------------------------------------------ NSA
def test_nsa_pipeline_small():
    """The 32K workload's head layout (16 query heads per KV head) at an
    oracle-sized length with a ragged last block, end to end; the combine
    stage also against the GPU's own branch outputs."""
    c = replace(configs.NSA_32K, S=2048 + 64, Hq=16, Hkv=1)
    x = inputs.nsa_inputs(c, seed=0, device=DEV)
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV, fuse_combine=False)
    plan.run(x["q"], x["k"], x["v"], x["z"])
    _sync()
    exact = _nsa_end_to_end(c, x, plan)
    out = On.combine(to_np(plan.o_cmp), to_np(plan.o_sel), to_np(plan.o_win), to_np(x["z"]))
    check_bf16(to_np(plan.out), out, "combine of the GPU branches")
    print(f"bit-exact index rows: {exact:.3f}")


def test_nsa_pipeline_head_dim_64():
    """Head dimension 64 (the block-score kernel's other instance) with a
    ragged last block and two KV groups, end to end."""
    c = replace(configs.NSA_32K, S=1500 + 37, Hq=8, Hkv=2, D=64)
    x = inputs.nsa_inputs(c, seed=5, device=DEV)
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV, fuse_combine=False)
    plan.run(x["q"], x["k"], x["v"], x["z"])
    _sync()
    exact = _nsa_end_to_end(c, x, plan)
    print(f"bit-exact index rows: {exact:.3f}")


@pytest.mark.parametrize("S,Hq,Hkv,window", [(2048 + 64, 16, 1, 512), (1000, 8, 2, 512),
                                              (777, 4, 1, 100)])
def test_nsa_window_combine_fused(S, Hq, Hkv, window):
    """Sliding branch with the gated combine in its epilogue: against the
    oracle's window branch combined with the GPU's other two branches, and
    against the two-call path (which rounds o_win to bf16 first)."""
    c = replace(configs.NSA_32K, S=S, Hq=Hq, Hkv=Hkv, window=window)
    x = inputs.nsa_inputs(c, seed=S, device=DEV)
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV, fuse_combine=False)
    plan.run(x["q"], x["k"], x["v"], x["z"])
    fused = torch.full_like(plan.out, float("nan"))
    L.dsa_nsa_window_combine(x["q"], x["k"], x["v"], c.window, c.scale, plan.o_cmp, plan.o_sel,
                             x["z"], fused)
    _sync()
    q, k, v, z = (to_np(x[n]) for n in ("q", "k", "v", "z"))
    o3, _ = On.window_attention(q, k, v, c.window, c.scale)
    ref = On.combine(to_np(plan.o_cmp), to_np(plan.o_sel), o3, z)
    check_bf16(to_np(fused), ref, "fused window + combine")
    check_bf16(to_np(fused), to_np(plan.out), "fused against two calls")


def _bits(t):
    return t.view(torch.int16).cpu()


@pytest.mark.parametrize("S,B,Hq,Hkv,window", [(2048 + 64, 1, 16, 1, 512), (1000, 1, 8, 2, 512),
                                                (777, 1, 4, 1, 100), (1100, 2, 8, 2, 512),
                                                (64, 1, 4, 1, 512), (37, 1, 4, 1, 16),
                                                (1000, 1, 16, 2, 256)])
def test_nsa_select_window_combine(S, B, Hq, Hkv, window):
    """The selected and sliding branches with the gated combine in one pass
    over each query block's rows: bit for bit the index-mode call followed by
    the fused window + combine, and end to end against the oracle (a plan
    that runs the fused pass, whose o_sel and o_win are never written)."""
    c = replace(configs.NSA_32K, B=B, S=S, Hq=Hq, Hkv=Hkv, window=window)
    x = inputs.nsa_inputs(c, seed=S + 7, device=DEV)
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV, fuse_branches=False)
    assert plan.fuse_combine and not plan.fuse_branches
    plan.run(x["q"], x["k"], x["v"], x["z"])
    one = torch.full_like(plan.out, float("nan"))
    L.dsa_nsa_select_window_combine(x["q"], x["k"], x["v"], plan.idx, plan.count, c.sel_block,
                                    c.window, c.scale, plan.o_cmp, x["z"], one)
    _sync()
    assert torch.equal(_bits(one), _bits(plan.out)), "one pass differs from the two calls"
    fplan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                    c.window, x["q"].dtype, DEV)
    assert fplan.fuse_branches
    fplan.run(x["q"], x["k"], x["v"], x["z"])
    _sync()
    assert torch.equal(_bits(fplan.out), _bits(one))
    q, k, v, z = (to_np(x[n]) for n in ("q", "k", "v", "z"))
    ref = On.forward(q, k, v, z, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k, c.window, c.scale,
                     summary_dtype="bf16")
    gi, gc = fplan.idx.cpu().numpy(), fplan.count.cpu().numpy()
    check_indices(ref["scores"], gi, gc, c.sel_k, 0, True)
    if np.array_equal(gi, ref["idx"]) and np.array_equal(gc, ref["count"]):
        full = ref["out"]
    else:   # accepted near-ties: the oracle's selected branch at the GPU's lists
        o2, _ = Op.sparse_attention(q, k, v, gi, gc, c.sel_block, c.scale)
        full = On.combine(ref["o_cmp"], o2, ref["o_win"], z)
    check_bf16(to_np(fplan.out), full, "one-pass selected + sliding + combine, end to end")


@pytest.mark.parametrize("S,Hq,Hkv,sel_k,window", [(1500, 8, 2, 6, 384), (1024, 4, 1, 4, 128)])
def test_nsa_select_window_combine_128_token_blocks(S, Hq, Hkv, sel_k, window):
    """The one pass with 128-token selection blocks (two key tiles per
    listed block; window tiles from 128-row query blocks) end to end against
    the oracle."""
    c = replace(configs.NSA_32K, S=S, Hq=Hq, Hkv=Hkv, sel_block=128, sel_k=sel_k, window=window)
    x = inputs.nsa_inputs(c, seed=S + 3, device=DEV)
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV)
    assert plan.fuse_branches
    plan.run(x["q"], x["k"], x["v"], x["z"])
    _sync()
    q, k, v, z = (to_np(x[n]) for n in ("q", "k", "v", "z"))
    ref = On.forward(q, k, v, z, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k, c.window, c.scale,
                     summary_dtype="bf16")
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    check_indices(ref["scores"], gi, gc, c.sel_k, 0, True)
    if np.array_equal(gi, ref["idx"]) and np.array_equal(gc, ref["count"]):
        full = ref["out"]
    else:
        o2, _ = Op.sparse_attention(q, k, v, gi, gc, c.sel_block, c.scale)
        full = On.combine(ref["o_cmp"], o2, ref["o_win"], z)
    check_bf16(to_np(plan.out), full, "one pass, 128-token blocks, end to end")


def test_nsa_select_window_combine_empty_lists():
    """Query blocks whose list is empty (count 0) take only the window pass
    (their selected output is zero), bit for bit as the two calls do."""
    c = replace(configs.NSA_32K, S=1000, Hq=8, Hkv=2)
    x = inputs.nsa_inputs(c, seed=11, device=DEV)
    plan = NSAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.cmp_len, c.cmp_stride, c.sel_block, c.sel_k,
                   c.window, x["q"].dtype, DEV, fuse_branches=False)
    plan.run(x["q"], x["k"], x["v"], x["z"])
    count = plan.count.clone()
    count[:, :, ::3] = 0
    count[:, 1, 5:9] = 0
    o_sel = torch.empty_like(plan.out)
    L.dsa_sparse_attn_prefill(x["q"], x["k"], x["v"], plan.idx, count, c.sel_block, 0, c.scale,
                              o_sel)
    two = torch.empty_like(plan.out)
    L.dsa_nsa_window_combine(x["q"], x["k"], x["v"], c.window, c.scale, plan.o_cmp, o_sel, x["z"],
                             two)
    one = torch.full_like(plan.out, float("nan"))
    L.dsa_nsa_select_window_combine(x["q"], x["k"], x["v"], plan.idx, count, c.sel_block,
                                    c.window, c.scale, plan.o_cmp, x["z"], one)
    _sync()
    assert (o_sel[:, :, :64].float() == 0).all()
    assert torch.equal(_bits(one), _bits(two))


def test_nsa_combine_only():
    rng = torch.Generator().manual_seed(0)
    o = [torch.randn(1, 4, 100, 128, generator=rng).to(torch.bfloat16) for _ in range(3)]
    z = torch.randn(1, 100, 4, 3, generator=rng)
    out = torch.empty_like(o[0], device=DEV)
    L.dsa_nsa_combine(*(t.to(DEV) for t in o), z.to(DEV), out)
    _sync()
    ref = On.combine(*(to_np(t) for t in o), z.numpy())
    check_bf16(to_np(out), ref, "combine")


def test_decode_repeated_calls_identical():
    """Repeated calls on one workspace give bit-identical outputs."""
    c = replace(configs.DECODE_128K, B=3, L=8192)
    x = inputs.decode_inputs(c, seed=7, device=DEV)
    plan = DecodePlan(c.B, c.Hq, c.Hkv, c.L, c.D, c.page, 9, x["q"].dtype, DEV)
    plan.build_metadata(x["k"])
    outs = []
    for _ in range(3):
        plan.run(x["q"], x["k"], x["v"])
        outs.append(plan.out.clone())
    _sync()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 16 * 37])
def test_read_stream_reads_every_word(nbytes):
    """The read-stream yardstick touches every word once: the XOR of its
    per-workgroup words equals the XOR of the buffer."""
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    n = L.load().dsa_read_stream_sink_words()
    sink = torch.zeros(n + 5, dtype=torch.int32, device=DEV)
    L.dsa_read_stream(src.to(DEV), sink)
    _sync()
    got = np.bitwise_xor.reduce(sink.cpu().numpy()[:n].view(np.uint32))
    want = np.bitwise_xor.reduce(src.numpy().view(np.uint32))
    assert got == want
    assert (sink.cpu().numpy()[n:] == 0).all()
