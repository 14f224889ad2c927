"""Work counters for throughput and roofline figures.

Plain arithmetic on shapes and selection counts; no tensors.  FLOPs count
2 per multiply-add and include both Q.K^T and P.V.
"""
from __future__ import annotations


def dense_pairs(n: int, causal: bool = False) -> int:
    """Query-key pairs of full attention over n tokens: n*n, or n(n+1)/2
    causally ([DMA] §二 and [SF] §一: cost grows with the square of length)."""
    return n * (n + 1) // 2 if causal else n * n


def prefill_selected_blocks(n_blocks: int, topk: int, n_local: int) -> int:
    """Sum over query blocks of the number of selected key blocks,
    min(i + 1, topk + n_local) for block i (causal selection + window)."""
    return sum(min(i + 1, topk + n_local) for i in range(n_blocks))


def prefill_effective_flops(Hq: int, D: int, block: int, selected_blocks: int, B: int = 1) -> float:
    """Work on the selected blocks only, each counted as a full
    block x block tile (the diagonal block included): 4*D*block^2 per
    (query head, selected block)."""
    return 4.0 * D * block * block * selected_blocks * Hq * B


def prefill_exact_pair_flops(Hq: int, D: int, pairs: int, B: int = 1) -> float:
    """4*D per visible (query, key) pair."""
    return 4.0 * D * pairs * Hq * B


def decode_selected_bytes(B: int, Hkv: int, pages_selected: int, page: int, D: int,
                          elem_bytes: int = 2) -> int:
    """K and V bytes of the selected pages: what one decode step must read."""
    return 2 * B * Hkv * pages_selected * page * D * elem_bytes


def prefill_attention_bytes(B, Hq, Hkv, S, D, elem_bytes=2, lse=True, idx_bytes=0) -> int:
    """Compulsory HBM traffic of the attention kernel: Q and O once, K and V
    once (re-reads hit cache), LSE and index lists."""
    return (2 * B * Hq * S * D + 2 * B * Hkv * S * D) * elem_bytes + (4 * B * Hq * S if lse else 0) + idx_bytes
