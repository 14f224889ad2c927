"""dsa_sparse_attn_decode_noalloc through the C ABI: the decode with the
library's per-device scratch in place of a workspace gives the same bits as
dsa_sparse_attn_decode on the same inputs and page lists, and meets the
output bar against the oracle; two calls in a row, the second smaller (the
scratch keeps the first call's contents)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from dynamic_block_sparse_head_amd import binding as L
from dynamic_block_sparse_head_amd import configs, inputs
from dynamic_block_sparse_head_amd.pipeline import DecodePlan
from oracle import decode as Od

from _parity import check_bf16, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_decode_noalloc_matches_workspace_call():
    cases = [(configs.DECODE_128K, configs.DECODE_128K.topk),            # the full 128K workload
             (replace(configs.DECODE_128K, B=3, L=4096, page=128), 7)]   # then a smaller one
    for c, topk in cases:
        print(f"noalloc decode: B={c.B} L={c.L} page={c.page} top {topk}", flush=True)
        x = inputs.decode_inputs(c, seed=c.B, device=DEV)
        plan = DecodePlan(c.B, c.Hq, c.Hkv, c.L, c.D, c.page, topk, x["q"].dtype, DEV)
        plan.build_metadata(x["k"])
        plan.run(x["q"], x["k"], x["v"])
        out = torch.full_like(plan.out, float("nan"))
        L.dsa_sparse_attn_decode_noalloc(x["q"], x["k"], x["v"], plan.idx, plan.count, c.page,
                                         c.scale, out)
        torch.cuda.synchronize()
        assert torch.equal(out, plan.out), "noalloc decode differs from the workspace call"
        # the output bar against the oracle, on sampled (sequence, KV head) rows
        gi, gc = plan.idx.cpu().numpy(), plan.count.cpu().numpy()
        for (b, g) in [(0, 0), (c.B - 1, c.Hkv - 1)]:
            heads = slice(g * c.G, (g + 1) * c.G)
            ref = Od.decode_attention(to_np(x["q"][b:b + 1, heads]), to_np(x["k"][b:b + 1, g:g + 1]),
                                      to_np(x["v"][b:b + 1, g:g + 1]), gi[b:b + 1, g:g + 1, 0],
                                      gc[b:b + 1, g:g + 1, 0], c.page, c.scale)
            check_bf16(to_np(out[b:b + 1, heads]), ref, f"noalloc decode b{b} g{g}")
        del x, plan
        torch.cuda.empty_cache()
