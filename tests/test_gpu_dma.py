"""GPU parity of the value-driven dynamic mask ([DMA] §四-§五): weights and
block scores, selection, and attention with each kept key's weight added to
its logit, against the float64 oracle."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from dynamic_block_sparse_head_amd import binding as L
from dynamic_block_sparse_head_amd import configs, inputs
from dynamic_block_sparse_head_amd.pipeline import DMAPlan
from oracle import dma as M
from oracle import prefill as Op

from _parity import check_bf16, check_f32, check_indices, check_lse, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
W_REL = 1e-5   # float32 dot (D terms), softplus and exp against float64


def _run(c, seed=0, plant=None):
    x = inputs.prefill_inputs(c, seed=seed, device=DEV)
    proj, gain = inputs.dma_params(c, seed=seed, device=DEV)
    v = x["v"]
    if plant is not None:   # values of block `plant` pushed along each head's projection
        d = proj / torch.linalg.vector_norm(proj, dim=1, keepdim=True)
        v = v.clone()
        v[:, :, plant * c.block:(plant + 1) * c.block] += (0.5 * d[None, :, None, :]).to(v.dtype)
    plan = DMAPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, x["q"].dtype, DEV)
    plan.run(x["q"], x["k"], v, proj, gain)
    torch.cuda.synchronize()
    q, k, vn = to_np(x["q"]), to_np(x["k"]), to_np(v)
    w_ref = M.dynamic_weights(vn, to_np(proj), to_np(gain))
    w = to_np(plan.weights)
    assert np.max(np.abs(w - w_ref) / w_ref) < W_REL
    s_ref = M.block_scores(w_ref, c.block)
    s = to_np(plan.scores)
    assert (np.isneginf(s) == np.isneginf(s_ref)).all()
    fin = np.isfinite(s_ref)
    assert np.max(np.abs(s[fin] - s_ref[fin]) / s_ref[fin]) < W_REL
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    exact = check_indices(s_ref, gi, gc, c.topk, c.n_local, True)
    out, lse = M.biased_sparse_attention(q, k, vn, gi, gc, c.block, c.scale, w_ref)
    if c.dtype == "f32":
        check_f32(to_np(plan.out), out, c.name)
        check_lse(to_np(plan.lse), lse, 1e-4, c.name)
    else:
        check_bf16(to_np(plan.out), out, c.name)
        check_lse(to_np(plan.lse), lse, 2e-3, c.name)
    return exact, gi, gc


@pytest.mark.parametrize("S", [2048, 2000])
def test_dma_16k_shape(S):
    exact, _, _ = _run(configs.PREFILL_16K.with_seq(S))
    assert exact > 0.9


def test_dma_batch_of_two():
    _run(replace(configs.PREFILL_16K.with_seq(1000), B=2), seed=7)


def test_dma_64k_shape():
    _run(configs.PREFILL_64K.with_seq(6144))


def test_dma_tiny_f32():
    _run(configs.TINY_F32)


def test_planted_heavy_block_kept():
    c = configs.PREFILL_16K.with_seq(2048)
    _, gi, gc = _run(c, seed=1, plant=5)
    for g in range(c.Hkv):
        for i in range(5 + c.n_local, c.n_blocks):
            assert 5 in gi[0, g, i, :gc[0, g, i]]


def test_constant_key_bias_shifts_lse_only():
    """A constant bias leaves the softmax weights unchanged and moves the
    log-sum-exp by exactly that constant."""
    c = configs.PREFILL_16K.with_seq(1024)
    x = inputs.prefill_inputs(c, seed=7, device=DEV)
    q, k, v = to_np(x["q"]), to_np(x["k"]), to_np(x["v"])
    s = Op.block_scores_pooled(q, k, c.block)
    idx, cnt = Op.select_blocks(s, c.topk, c.n_local, True)
    idx_d, cnt_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV)
    bias = torch.full((c.B, c.Hkv, c.S), 1.75, dtype=torch.float32, device=DEV)
    out = torch.empty_like(x["q"])
    lse = torch.empty((c.B, c.Hq, c.S), dtype=torch.float32, device=DEV)
    L.dsa_sparse_attn_prefill_ex(x["q"], x["k"], x["v"], idx_d, cnt_d, c.block, c.G, bias, c.scale,
                                 out, lse)
    torch.cuda.synchronize()
    ref, rl = Op.sparse_attention(q, k, v, idx, cnt, c.block, c.scale)
    check_bf16(to_np(out), ref, "constant bias")
    check_lse(to_np(lse), rl + 1.75, 2e-3, "constant bias")
