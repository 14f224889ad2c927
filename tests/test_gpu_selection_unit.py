"""GPU parity of the per-query-head selection variant (every query head of a
KV group ranks blocks by its own pooled score and keeps its own index list)
and of index lists shared by an arbitrary number of heads (sel_heads),
against the float64 oracle."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from dynamic_block_sparse_head_amd import binding as L
from dynamic_block_sparse_head_amd import configs, inputs
from dynamic_block_sparse_head_amd.pipeline import PrefillPlan
from oracle import prefill as Op

from _parity import check_bf16, check_f32, check_indices, check_lse, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _per_head(c, seed=0):
    x = inputs.prefill_inputs(c, seed=seed, device=DEV)
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, x["q"].dtype, DEV,
                       per_head=True)
    plan.run(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    q, k, v = to_np(x["q"]), to_np(x["k"]), to_np(x["v"])
    s_ref = Op.block_scores_pooled(q, k, c.block, sel_heads=1)
    got = to_np(plan.scores)
    assert got.shape == s_ref.shape
    assert (np.isneginf(got) == np.isneginf(s_ref)).all()
    fin = np.isfinite(s_ref)
    assert (np.abs(got[fin] - s_ref[fin]) <= 2.0 ** -23 * np.abs(s_ref[fin]) + 1e-30).all()
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    exact = check_indices(s_ref, gi, gc, c.topk, c.n_local, True)
    out, lse = Op.sparse_attention(q, k, v, gi, gc, c.block, c.scale, sel_heads=1)
    if c.dtype == "f32":
        check_f32(to_np(plan.out), out, c.name)
        check_lse(to_np(plan.lse), lse, 1e-4, c.name)
    else:
        check_bf16(to_np(plan.out), out, c.name)
        check_lse(to_np(plan.lse), lse, 2e-3, c.name)
    # the heads of a group really do choose differently (when there is a choice)
    B, Hq, nb, W = gi.shape
    grp = gi.reshape(B, c.Hkv, c.G, nb, W)
    assert c.G == 1 or nb <= c.topk + c.n_local or (grp != grp[:, :, :1]).any()
    return exact


@pytest.mark.parametrize("S", [2048, 2000])
def test_per_head_16k_shape(S):
    assert _per_head(configs.PREFILL_16K.with_seq(S)) > 0.99


def test_per_head_batch_of_two():
    _per_head(replace(configs.PREFILL_16K.with_seq(1000), B=2), seed=8)


def test_per_head_64k_shape_mixture():
    _per_head(configs.PREFILL_64K.with_seq(6144 - 64))


def test_per_head_block32_d64():
    c = replace(configs.PREFILL_16K, name="b32d64", S=1024 + 32, D=64, block=32, topk=5, window=64,
                q_std=0.125, kv_std=0.125, v_std=0.125, needles=2, needle_alpha=0.5)
    _per_head(c)


def test_per_head_tiny_f32():
    assert _per_head(configs.TINY_F32) == 1.0


@pytest.mark.parametrize("sel", [2, 4])
def test_lists_shared_by_sel_heads(sel):
    """Index lists given per unit of `sel` heads (chosen here by the oracle
    from its own scores): the attention follows them exactly."""
    c = configs.PREFILL_16K.with_seq(1024 + 64)
    x = inputs.prefill_inputs(c, seed=2, device=DEV)
    q, k, v = to_np(x["q"]), to_np(x["k"]), to_np(x["v"])
    s = Op.block_scores_pooled(q, k, c.block, sel_heads=sel)
    idx, cnt = Op.select_blocks(s, c.topk, c.n_local, True)
    out = torch.empty_like(x["q"])
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device=DEV)
    L.dsa_sparse_attn_prefill_ex(x["q"], x["k"], x["v"], torch.from_numpy(idx).to(DEV),
                                 torch.from_numpy(cnt).to(DEV), c.block, sel, None, c.scale, out, lse)
    torch.cuda.synchronize()
    ref, rl = Op.sparse_attention(q, k, v, idx, cnt, c.block, c.scale, sel_heads=sel)
    check_bf16(to_np(out), ref, f"sel {sel}")
    check_lse(to_np(lse), rl, 2e-3, f"sel {sel}")


def test_sel_heads_equal_to_group_matches_the_group_call():
    c = configs.PREFILL_16K.with_seq(1024)
    x = inputs.prefill_inputs(c, seed=6, device=DEV)
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, x["q"].dtype, DEV)
    plan.run(x["q"], x["k"], x["v"])
    out = torch.empty_like(plan.out)
    L.dsa_sparse_attn_prefill_ex(x["q"], x["k"], x["v"], plan.idx, plan.count, c.block, c.G, None,
                                 c.scale, out)
    torch.cuda.synchronize()
    assert torch.equal(out, plan.out)
