"""GPU parity of the block-sparse attention backward (dq, dk, dv) against the
float64 oracle, evaluated at the index lists the GPU forward selected (the
forward's own parity tests cover those).  Cases: the 16K and 64K workload
shapes at oracle-sized lengths, ragged tails, D = 64, blocks of 32 and 256,
no grouping (Hq = Hkv), dense selection against autograd of plain causal
attention, keys no row sees, determinism and a zero upstream gradient."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from dynamic_block_sparse_head_amd import configs, inputs
from dynamic_block_sparse_head_amd.pipeline import PrefillPlan
from oracle import backward as Ob

from _parity import check_grad, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _forward_backward(c, seed=0, topk=None, n_local=None):
    x = inputs.prefill_inputs(c, seed=seed, device=DEV)
    dout = inputs.grad_output(c, seed=seed, device=DEV)
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block,
                       c.topk if topk is None else topk,
                       c.n_local if n_local is None else n_local, x["q"].dtype, DEV)
    plan.run(x["q"], x["k"], x["v"])
    dq, dk, dv = plan.backward(x["q"], x["k"], x["v"], dout)
    torch.cuda.synchronize()
    return x, dout, plan, (to_np(dq), to_np(dk), to_np(dv))


def _unseen_keys(gi, gc, block, S):
    """[B,Hkv,S] bool: keys in no selected block (so no row sees them)."""
    B, Hkv, nb, _ = gi.shape
    seen = np.zeros((B, Hkv, nb), dtype=bool)
    for b in range(B):
        for g in range(Hkv):
            for i in range(nb):
                seen[b, g, gi[b, g, i, :gc[b, g, i]]] = True
    return ~np.repeat(seen, block, axis=2)[:, :, :S]


def _parity(c, seed=0, **kw):
    x, dout, plan, got = _forward_backward(c, seed, **kw)
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    ref = Ob.sparse_attention_backward(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), gi, gc,
                                       c.block, c.scale, to_np(dout))
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        m, n = check_grad(g, r, f"{c.name} {name}")
        print(f"{c.name} {name}: max err / max|ref| {m:.2e}, norm err {n:.2e}")
    unseen = _unseen_keys(gi, gc, c.block, c.S)
    for name, g in (("dk", got[1]), ("dv", got[2])):
        assert (g[unseen] == 0).all(), f"{name}: nonzero gradient on keys no row sees"
    return unseen.mean()


@pytest.mark.parametrize("S", [2048, 2000])
def test_backward_16k_shape(S):
    _parity(configs.PREFILL_16K.with_seq(S))


def test_backward_16k_full_size_two_groups():
    """The 16K workload at full length, in the configuration the benchmark
    times (same plan, seed and upstream gradient): dq of every query head of
    KV groups 0 and 5, and dk, dv of those groups, against the float64
    oracle over the whole sequence; keys no row of a group sees get zero."""
    c = configs.PREFILL_16K
    x, dout, plan, got = _forward_backward(c, seed=0)
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    unseen = _unseen_keys(gi, gc, c.block, c.S)
    for g in (0, 5):
        heads = slice(g * c.G, (g + 1) * c.G)
        ref = Ob.sparse_attention_backward(
            to_np(x["q"][:, heads]), to_np(x["k"][:, g:g + 1]), to_np(x["v"][:, g:g + 1]),
            gi[:, g:g + 1], gc[:, g:g + 1], c.block, c.scale, to_np(dout[:, heads]))
        mine = (got[0][:, heads], got[1][:, g:g + 1], got[2][:, g:g + 1])
        for name, gg, r in zip(("dq", "dk", "dv"), mine, ref):
            m, n = check_grad(gg, r, f"16K g{g} {name}")
            print(f"16K g{g} {name}: max err / max|ref| {m:.2e}, norm err {n:.2e}")
        for name, gg in (("dk", mine[1]), ("dv", mine[2])):
            assert (gg[unseen[:, g:g + 1]] == 0).all(), f"{name}: nonzero gradient on unseen keys"


@pytest.mark.parametrize("S", [37, 65])
def test_backward_short_sequences(S):
    _parity(replace(configs.PREFILL_16K.with_seq(S), needles=0), seed=S)


def test_backward_single_token():
    """S = 1: the row's only key is itself, p = 1, so dS = p (dP - D) is zero
    in exact arithmetic (dout.v - dout.out with out = v) and dq, dk hold only
    the rounding of the two float32 dot products; dv = dout."""
    c = replace(configs.PREFILL_16K.with_seq(1), needles=0)
    x, dout, plan, got = _forward_backward(c, seed=1)
    gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
    ref = Ob.sparse_attention_backward(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), gi, gc,
                                       c.block, c.scale, to_np(dout))
    assert (ref[0] == 0).all() and (ref[1] == 0).all()
    # |dout| |v| over D = 128 terms, each product exact in float32: the two
    # sums differ by at most ~D * 2^-24 * sum|dout v|; scaled by 1/sqrt(D) |k|
    bound = 2.0 ** -16 * np.abs(to_np(dout)).max() * np.abs(to_np(x["v"])).max() * \
        np.abs(to_np(x["k"])).max() * c.D
    assert np.abs(got[0]).max() <= bound and np.abs(got[1]).max() <= bound
    check_grad(got[2], ref[2], f"{c.name} dv")


def test_backward_batch_of_two():
    """Two sequences: the staged D = 128 kernels and the generic ones."""
    _parity(replace(configs.PREFILL_16K.with_seq(1000), B=2), seed=5)
    _parity(replace(configs.PREFILL_16K, name="b32d64", B=2, S=600, D=64, block=32, topk=4,
                    window=64, q_std=0.125, kv_std=0.125, v_std=0.125, needles=2,
                    needle_alpha=0.5), seed=6)


def test_backward_64k_shape_mixture_ragged():
    _parity(configs.PREFILL_64K.with_seq(6080))


def test_backward_block32_d64():
    c = replace(configs.PREFILL_16K, name="b32d64", S=1024 + 32, D=64, block=32, topk=5, window=64,
                q_std=0.125, kv_std=0.125, v_std=0.125, needles=2, needle_alpha=0.5)
    _parity(c)


def test_backward_unseen_keys_get_zero():
    """No local window and k = 2: most key blocks are never selected, and
    their keys must get exactly zero dk and dv."""
    frac = _parity(configs.PREFILL_16K.with_seq(1024), topk=2, n_local=0)
    assert frac > 0


@pytest.mark.parametrize("D", [128, 64])
def test_backward_block256(D):
    c = replace(configs.PREFILL_16K, name=f"b256d{D}", S=2048 + 100, D=D, block=256, topk=2,
                window=256, needles=1)
    _parity(c)


def test_backward_no_grouping():
    c = replace(configs.PREFILL_16K, name="g1", Hq=4, Hkv=4, S=700, block=32, topk=4, window=64,
                needles=1)
    _parity(c)


def test_backward_dense_selection_matches_autograd():
    """Every block selected: the gradients of plain causal attention."""
    c = replace(configs.PREFILL_16K.with_seq(512), Hq=8, Hkv=2)
    x, dout, plan, got = _forward_backward(c, seed=4, topk=c.n_blocks, n_local=1)
    assert (plan.count.cpu().numpy() == np.arange(1, c.n_blocks + 1)).all()
    q, k, v = (torch.from_numpy(to_np(x[n])).requires_grad_() for n in "qkv")
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(c.G, 1), v.repeat_interleave(c.G, 1), is_causal=True, scale=c.scale)
    o.backward(torch.from_numpy(to_np(dout)))
    for name, g, r in zip(("dq", "dk", "dv"), got, (q.grad, k.grad, v.grad)):
        check_grad(g, r.numpy(), f"dense {name}")


def test_backward_deterministic_and_zero_grad():
    c = configs.PREFILL_16K.with_seq(1024)
    x = inputs.prefill_inputs(c, seed=2, device=DEV)
    dout = inputs.grad_output(c, seed=2, device=DEV)
    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, x["q"].dtype, DEV)
    plan.run(x["q"], x["k"], x["v"])
    first = [t.clone() for t in plan.backward(x["q"], x["k"], x["v"], dout)]
    second = plan.backward(x["q"], x["k"], x["v"], dout)
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a, b)
    for t in plan.backward(x["q"], x["k"], x["v"], torch.zeros_like(dout)):
        assert (t == 0).all()
