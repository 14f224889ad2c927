"""Seeded synthetic inputs for every workload.

This module only draws and shapes random tensors.  It holds none of the
method's arithmetic (no pooling, scoring, selection or softmax): both the
HIP path and the CPU oracle receive the very tensors made here, so the two
sides always see identical bits.

Values are drawn in float32 with a torch generator on the requested device
and rounded once to the workload's dtype (bfloat16 rounding is
round-to-nearest-even).  Integer choices (needle positions, cluster ids)
come from a numpy generator on the host, so they do not depend on the device.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import DecodeConfig, NSAConfig, PrefillConfig

_TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "gates": 3, "needles": 4, "clusters": 5, "dout": 6,
               "dma": 7}


def _dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _seed(seed: int, tag: str, tensor: str) -> int:
    base = sum((i + 1) * ord(ch) for i, ch in enumerate(tag))
    return (seed * 1_000_003 + base * 7919 + _TENSOR_IDS[tensor] * 104_729) % (2**62)


def _gen(device, seed: int, tag: str, tensor: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tag, tensor))
    return g


def _normal(shape, std, gen, device, chunk_dim0=True) -> torch.Tensor:
    """float32 N(0, std^2); drawn slice by slice along dim 0 to bound temp memory."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    if chunk_dim0 and len(shape) > 1 and shape[0] > 1:
        for i in range(shape[0]):
            out[i].normal_(0.0, std, generator=gen)
    else:
        out.normal_(0.0, std, generator=gen)
    return out


def _host_rng(seed: int, tag: str, tensor: str) -> np.random.Generator:
    return np.random.default_rng(_seed(seed, tag, tensor))


def _needle_plan(tag, B, Hkv, n_blocks, n_local, topk, needles, target_range, seed):
    """(b, g, target_query_block, needle_key_block) for `needles` needles per
    KV head: each needle block lies before its target's n_local most recent
    blocks (so it is a top-k candidate of the target) and the targets and
    needles of one KV head are all distinct blocks.  A sequence too short to
    hold them gets fewer (or none)."""
    if needles == 0:
        return []
    rng = _host_rng(seed, tag, "needles")
    nB, nl = n_blocks, n_local
    out = []
    for b in range(B):
        for g in range(Hkv):
            used = set()
            for _ in range(needles):
                for _attempt in range(1000):
                    if target_range:
                        lo, hi = target_range
                    else:
                        lo, hi = min(nl + topk + 8, nB - 1), nB - 1
                    t = int(rng.integers(lo, hi + 1))
                    last_cand = t - nl
                    if last_cand < 0:
                        continue
                    n = int(rng.integers(0, last_cand + 1))
                    if t in used or n in used or t == n:
                        continue
                    used.update((t, n))
                    out.append((b, g, t, n))
                    break
                else:
                    break   # no room left on this KV head
    return out


def plan_needles(cfg: PrefillConfig, seed: int):
    """Needles of a prefill workload: candidates of a target lie before its
    local window."""
    return _needle_plan(cfg.name, cfg.B, cfg.Hkv, cfg.n_blocks, cfg.n_local, cfg.topk, cfg.needles,
                        cfg.needle_target_range, seed)


def plan_nsa_needles(cfg: NSAConfig, seed: int):
    """Needles of a three-branch workload: every block up to the target is a
    candidate; a needle is kept off the target block itself."""
    return _needle_plan(cfg.name, cfg.B, cfg.Hkv, cfg.n_blocks, 1, cfg.sel_k, cfg.needles, (), seed)


def _plant(q, k, needles, G, blk, alpha):
    """Shift every key of each needle block by alpha along the unit direction
    of the summed query rows of its target block (all query heads of the KV
    group), so the needle lines up with what the target block asks for.
    q in its final dtype, k in float32 before rounding (modified in place)."""
    D = q.shape[-1]
    for (b, g, t, n) in needles:
        rows = q[b, g * G:(g + 1) * G, t * blk:(t + 1) * blk, :].to(torch.float64)
        direction = rows.reshape(-1, D).sum(dim=0)
        direction = direction / torch.linalg.vector_norm(direction)
        k[b, g, n * blk:(n + 1) * blk, :] += (alpha * direction).to(torch.float32)


def prefill_inputs(cfg: PrefillConfig, seed: int = 0, device="cpu"):
    """Q [B,Hq,S,D], K/V [B,Hkv,S,D] in cfg.dtype, plus the needle plan.

    Needles: every key of the needle block is shifted by needle_alpha along
    the unit direction of the summed query rows of the target block (all
    query heads of the KV group), so the needle block lines up with what the
    target block asks for.
    """
    dev = torch.device(device)
    B, Hq, Hkv, S, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.D
    q = _normal((B, Hq, S, D), cfg.q_std, _gen(dev, seed, cfg.name, "q"), dev)
    if cfg.keys == "mixture":
        rng = _host_rng(seed, cfg.name, "clusters")
        gk = _gen(dev, seed, cfg.name, "k")
        k = torch.empty((B, Hkv, S, D), dtype=torch.float32, device=dev)
        nB = cfg.n_blocks
        for b in range(B):
            for g in range(Hkv):
                centres = torch.empty((cfg.n_clusters, D), dtype=torch.float32, device=dev)
                centres.normal_(0.0, 1.0, generator=gk)
                ids = torch.as_tensor(rng.integers(0, cfg.n_clusters, size=nB), device=dev)
                per_tok = ids.repeat_interleave(cfg.block)[:S]
                eps = torch.empty((S, D), dtype=torch.float32, device=dev)
                eps.normal_(0.0, 1.0, generator=gk)
                k[b, g] = (centres[per_tok] + eps) * cfg.kv_std
    else:
        k = _normal((B, Hkv, S, D), cfg.kv_std, _gen(dev, seed, cfg.name, "k"), dev)
    v = _normal((B, Hkv, S, D), cfg.v_std, _gen(dev, seed, cfg.name, "v"), dev)

    dt = _dtype(cfg.dtype)
    q = q.to(dt)
    needles = plan_needles(cfg, seed)
    _plant(q, k, needles, cfg.G, cfg.block, cfg.needle_alpha)
    return {"q": q.contiguous(), "k": k.to(dt).contiguous(), "v": v.to(dt).contiguous(),
            "needles": needles}


def grad_output(cfg: PrefillConfig, seed: int = 0, device="cpu"):
    """Upstream gradient dout [B,Hq,S,D] ~ N(0,1) in cfg.dtype, for the backward."""
    dev = torch.device(device)
    d = _normal((cfg.B, cfg.Hq, cfg.S, cfg.D), 1.0, _gen(dev, seed, cfg.name, "dout"), dev)
    return d.to(_dtype(cfg.dtype)).contiguous()


def dma_params(cfg: PrefillConfig, seed: int = 0, device="cpu"):
    """Value-driven mask parameters per KV head: a projection Delta [Hkv,D]
    ~ N(0, 1/(D v_std^2)), so that v . Delta ~ N(0, 1) whatever the value
    scale, and a gain A [Hkv] ~ U(0.1, 0.5), both float32."""
    rng = _host_rng(seed, cfg.name, "dma")
    delta = (rng.standard_normal((cfg.Hkv, cfg.D)) / (np.sqrt(cfg.D) * cfg.v_std)).astype(np.float32)
    A = rng.uniform(0.1, 0.5, size=cfg.Hkv).astype(np.float32)
    return torch.from_numpy(delta).to(device), torch.from_numpy(A).to(device)


def decode_inputs(cfg: DecodeConfig, seed: int = 0, device="cpu"):
    """q [B,Hq,D]; K/V cache [B,Hkv,L,D]; all N(0,1) in cfg.dtype."""
    dev = torch.device(device)
    dt = _dtype(cfg.dtype)
    q = _normal((cfg.B, cfg.Hq, cfg.D), 1.0, _gen(dev, seed, cfg.name, "q"), dev).to(dt)
    out = {"q": q.contiguous()}
    for name in ("k", "v"):
        gen = _gen(dev, seed, cfg.name, name)
        t = torch.empty((cfg.B, cfg.Hkv, cfg.L, cfg.D), dtype=dt, device=dev)
        for b in range(cfg.B):
            t[b] = _normal((cfg.Hkv, cfg.L, cfg.D), 1.0, gen, dev).to(dt)
        out[name] = t
    return out


def nsa_inputs(cfg: NSAConfig, seed: int = 0, device="cpu", needle_alpha=None):
    """Q [B,Hq,S,D], K/V [B,Hkv,S,D] ~ N(0, std^2) in cfg.dtype; gate logits
    z [B,S,Hq,3] ~ N(0,1) float32.  With cfg.needles > 0, needle blocks are
    planted in K as for the prefill workloads (sel_block-token blocks,
    strength needle_alpha, default cfg.needle_alpha); the draws do not depend
    on the strength, so one seed gives the same tensors at every alpha."""
    dev = torch.device(device)
    dt = _dtype(cfg.dtype)
    q = _normal((cfg.B, cfg.Hq, cfg.S, cfg.D), cfg.std, _gen(dev, seed, cfg.name, "q"), dev)
    k = _normal((cfg.B, cfg.Hkv, cfg.S, cfg.D), cfg.std, _gen(dev, seed, cfg.name, "k"), dev)
    v = _normal((cfg.B, cfg.Hkv, cfg.S, cfg.D), cfg.std, _gen(dev, seed, cfg.name, "v"), dev)
    z = _normal((cfg.B, cfg.S, cfg.Hq, 3), 1.0, _gen(dev, seed, cfg.name, "gates"), dev)
    q = q.to(dt)
    needles = plan_nsa_needles(cfg, seed)
    alpha = cfg.needle_alpha if needle_alpha is None else needle_alpha
    _plant(q, k, needles, cfg.G, cfg.sel_block, alpha)
    return {"q": q.contiguous(), "k": k.to(dt).contiguous(),
            "v": v.to(dt).contiguous(), "z": z.contiguous(), "needles": needles}


def random_scores(rows: int, n: int, seed: int = 0, ties: bool = False, device="cpu"):
    """float32 score rows for exercising selection alone.  With ties=True the
    values are drawn from a small set so exact ties are common."""
    rng = _host_rng(seed, "scores", "q")
    if ties:
        s = rng.integers(0, 7, size=(rows, n)).astype(np.float32) * np.float32(0.25)
    else:
        s = rng.standard_normal((rows, n)).astype(np.float32)
    return torch.from_numpy(s).to(device)
