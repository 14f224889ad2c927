"""The five workloads of the library, as plain data.

Every concrete parameter below (block sizes, k, windows, compression stride)
comes from the workload descriptions this library is built for; the pages
that describe the method name none of them.  Readings of points those
descriptions leave open are named fields, so every test and benchmark uses
the same values.

Page key used in citations:
  [DMA]  lsdiaocha.cn/2025/0807/3170092.shtml, a retelling of
         "Dynamic Mask Attention" (arXiv:2508.02124).
  [SA]   studyai.ink/2025/08/30 "什么是稀疏注意力" (sparse-attention explainer).
  [NSA]  news.news/tag/稀疏注意力, a summary of "Native Sparse Attention".
  [SF]   techwalker.com/2025/0429/3165971.shtml, a retelling of
         "The Sparse Frontier" (arXiv:2504.17768).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class PrefillConfig:
    """Causal top-k block-sparse prefill ([DMA] §四-§五, [SF] §二 block-sparse).

    window is in tokens and is a whole number of blocks, so the window is
    the n_local = window // block most recent key blocks, diagonal included.
    """
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    block: int
    topk: int
    window: int
    dtype: str            # "f32" or "bf16"
    q_std: float          # Q ~ N(0, q_std^2)
    kv_std: float         # K (and V unless v_std given) ~ N(0, kv_std^2)
    v_std: float
    keys: str = "normal"  # "normal" | "mixture"
    n_clusters: int = 0   # mixture: cluster id drawn per key block
    needles: int = 0      # planted needle blocks per KV head
    needle_alpha: float = 0.0
    needle_target_range: tuple = ()   # inclusive range of target query blocks (c1)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_blocks(self) -> int:
        return -(-self.S // self.block)

    @property
    def n_local(self) -> int:
        return self.window // self.block

    @property
    def sel_width(self) -> int:
        return self.topk + self.n_local

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def with_seq(self, S: int, name: str | None = None) -> "PrefillConfig":
        """Same workload at another sequence length (for oracle-sized tests)."""
        from dataclasses import replace
        return replace(self, S=S, name=name or f"{self.name}@S{S}")


@dataclass(frozen=True)
class DecodeConfig:
    """Single-token decode with page selection from per-page key bounds
    ([SF] §二-§四: page-level selection, whole KV cache kept)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    D: int
    page: int
    dtype: str = "bf16"
    compression: int = 20   # keep 1/compression of the pages ([SF] §三)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_pages(self) -> int:
        return self.L // self.page

    @property
    def topk(self) -> int:
        return self.n_pages // self.compression

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


@dataclass(frozen=True)
class NSAConfig:
    """Three-branch attention: compressed, selected, sliding; sigmoid-gated
    per token and head ([NSA] §03)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    cmp_len: int = 32
    cmp_stride: int = 16
    sel_block: int = 64
    sel_k: int = 16
    window: int = 512
    dtype: str = "bf16"
    std: float = 1.0 / math.sqrt(128)
    needles: int = 0          # planted needle blocks per KV head (parity runs only)
    needle_alpha: float = 0.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_cmp(self) -> int:
        return (self.S - self.cmp_len) // self.cmp_stride + 1 if self.S >= self.cmp_len else 0

    @property
    def n_blocks(self) -> int:
        return -(-self.S // self.sel_block)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def with_seq(self, S: int, name: str | None = None) -> "NSAConfig":
        from dataclasses import replace
        return replace(self, S=S, name=name or f"{self.name}@S{S}")


TINY_F32 = PrefillConfig(
    name="tiny_f32_prefill", B=1, Hq=2, Hkv=2, S=256, D=64, block=32, topk=2,
    window=32, dtype="f32", q_std=1.0, kv_std=1.0, v_std=1.0,
    needles=1, needle_alpha=2.0, needle_target_range=(3, 7))

PREFILL_16K = PrefillConfig(
    name="bf16_prefill_16k", B=1, Hq=32, Hkv=8, S=16384, D=128, block=64,
    topk=16, window=512, dtype="bf16", q_std=1 / math.sqrt(128),
    kv_std=1 / math.sqrt(128), v_std=1 / math.sqrt(128),
    needles=4, needle_alpha=0.25 * (1 / math.sqrt(128)) * math.sqrt(128))

PREFILL_64K = PrefillConfig(
    name="bf16_prefill_64k_mixture", B=1, Hq=32, Hkv=8, S=65536, D=128,
    block=128, topk=32, window=1024, dtype="bf16", q_std=1 / math.sqrt(128),
    kv_std=1 / math.sqrt(128), v_std=1.0, keys="mixture", n_clusters=8)

DECODE_128K = DecodeConfig(
    name="bf16_decode_128k_pages", B=16, Hq=32, Hkv=8, L=131072, D=128, page=64)

NSA_32K = NSAConfig(name="bf16_nsa_32k", B=1, Hq=64, Hkv=4, S=32768, D=128)

ALL = {c.name: c for c in (TINY_F32, PREFILL_16K, PREFILL_64K, DECODE_128K, NSA_32K)}
