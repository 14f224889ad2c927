"""HIP-graph replay of whole steps gives the eager results, replay after
replay, with other eager work and synchronizations in between."""
import pytest
import torch

from dynamic_block_sparse_head_amd import configs, inputs
from dynamic_block_sparse_head_amd.pipeline import DecodePlan, GraphedStep, PrefillPlan

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_prefill_step_graph_replays_match_eager():
    c = configs.PREFILL_16K.with_seq(2048 + 64)
    x = inputs.prefill_inputs(c, seed=3, device=DEV)
    other = inputs.prefill_inputs(c, seed=4, device=DEV)
    eager = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, x["q"].dtype, DEV)
    eager.run(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    want = (eager.out.clone(), eager.lse.clone(), eager.idx.clone(), eager.count.clone())

    plan = PrefillPlan(c.B, c.Hq, c.Hkv, c.S, c.D, c.block, c.topk, c.n_local, x["q"].dtype, DEV)
    step = GraphedStep(lambda: plan.run(x["q"], x["k"], x["v"]))
    for rep in range(3):
        plan.out.zero_()
        plan.lse.zero_()
        step()
        torch.cuda.synchronize()
        got = (plan.out, plan.lse, plan.idx, plan.count)
        for g, w in zip(got, want):
            assert torch.equal(g, w), f"replay {rep}"
        eager.run(other["q"], other["k"], other["v"])   # unrelated eager work between replays
        torch.cuda.synchronize()


def test_decode_step_graph_replays_match_eager():
    c = configs.DECODE_128K.__class__(**{**configs.DECODE_128K.__dict__, "B": 2, "L": 8192})
    x = inputs.decode_inputs(c, seed=5, device=DEV)
    eager = DecodePlan(c.B, c.Hq, c.Hkv, c.L, c.D, c.page, c.topk, x["q"].dtype, DEV)
    eager.build_metadata(x["k"])
    plan = DecodePlan(c.B, c.Hq, c.Hkv, c.L, c.D, c.page, c.topk, x["q"].dtype, DEV)
    plan.build_metadata(x["k"])
    q = x["q"].clone()
    step = GraphedStep(lambda: plan.run(q, x["k"], x["v"]))
    for rep, seed in enumerate([6, 7, 8]):
        qn = inputs.decode_inputs(c.__class__(**{**c.__dict__, "L": c.page}), seed=seed, device=DEV)["q"]
        q.copy_(qn)
        step()
        eager.run(qn, x["k"], x["v"])
        torch.cuda.synchronize()
        assert torch.equal(plan.idx, eager.idx), f"replay {rep}"
        assert torch.equal(plan.out, eager.out), f"replay {rep}"
