"""The three paths as sequences of library calls.

Orchestration only: outputs and workspaces are allocated with torch (device
memory), every step is a call into libdsa.so on the current stream.  Plans
allocate once so that repeated runs (benchmarks, serving loops) allocate
nothing.
"""
from __future__ import annotations

import math

import torch

from . import binding as L


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


class PrefillPlan:
    """Pooled scores -> top-k + window -> block-sparse attention ([DMA] §五).

    per_head=False: one selection per KV group (its query heads' scores
    summed); per_head=True: every query head ranks and keeps its own blocks."""

    def __init__(self, B, Hq, Hkv, S, D, block, topk, n_local, dtype, device, scale=None,
                 per_head=False):
        self.B, self.Hq, self.Hkv, self.S, self.D = B, Hq, Hkv, S, D
        self.block, self.topk, self.n_local = block, topk, n_local
        self.scale = scale if scale is not None else 1.0 / math.sqrt(D)
        self.nb = -(-S // block)
        self.per_head = per_head
        self.kind = L.DSA_SCORE_POOLED_HEAD if per_head else L.DSA_SCORE_POOLED
        U = Hq if per_head else Hkv                     # selection units per sequence
        ws = L.dsa_block_scores_workspace_size(self.kind, B, Hq, Hkv, S, D, block)
        self.ws = _empty((ws,), torch.uint8, device)
        self.scores = _empty((B, U, self.nb, self.nb), torch.float32, device)
        self.idx = _empty((B, U, self.nb, topk + n_local), torch.int32, device)
        self.count = _empty((B, U, self.nb), torch.int32, device)
        self.out = _empty((B, Hq, S, D), dtype, device)
        self.lse = _empty((B, Hq, S), torch.float32, device)

    def score(self, q, k):
        L.dsa_block_scores(self.kind, q, k, None, self.block, self.ws, self.scores)

    def select(self):
        L.dsa_topk_select(self.scores, self.topk, self.n_local, True, self.idx, self.count)

    def attend(self, q, k, v):
        if self.per_head:
            L.dsa_sparse_attn_prefill_ex(q, k, v, self.idx, self.count, self.block, 1, None,
                                         self.scale, self.out, self.lse)
        else:
            L.dsa_sparse_attn_prefill(q, k, v, self.idx, self.count, self.block, 0, self.scale,
                                      self.out, self.lse)

    def run(self, q, k, v):
        self.score(q, k)
        self.select()
        self.attend(q, k, v)
        return self.out

    def backward(self, q, k, v, dout):
        """dq, dk, dv of the last run's attention for the upstream gradient
        dout ([DMA] §四-§五); the run's index lists are held fixed.  Takes
        per-KV-group lists only."""
        if self.per_head:
            raise NotImplementedError("the backward takes per-KV-group index lists")
        if not hasattr(self, "dq"):
            B, Hq, Hkv, S, D = self.B, self.Hq, self.Hkv, self.S, self.D
            ws = L.dsa_sparse_attn_prefill_backward_workspace_size(B, Hq, Hkv, S, D, self.block)
            self.bwd_ws = _empty((ws,), torch.uint8, q.device)
            self.dq = _empty((B, Hq, S, D), q.dtype, q.device)
            self.dk = _empty((B, Hkv, S, D), q.dtype, q.device)
            self.dv = _empty((B, Hkv, S, D), q.dtype, q.device)
        L.dsa_sparse_attn_prefill_backward(q, k, v, self.out, self.lse, dout, self.idx, self.count,
                                           self.block, self.scale, self.bwd_ws, self.dq, self.dk,
                                           self.dv)
        return self.dq, self.dk, self.dv


class DMAPlan:
    """Value-driven dynamic mask ([DMA] §四-§五): weights from the values ->
    heaviest key blocks + window -> attention over them with each kept key's
    weight added to its logit."""

    def __init__(self, B, Hq, Hkv, S, D, block, topk, n_local, dtype, device, scale=None):
        self.B, self.Hq, self.Hkv, self.S, self.D = B, Hq, Hkv, S, D
        self.block, self.topk, self.n_local = block, topk, n_local
        self.scale = scale if scale is not None else 1.0 / math.sqrt(D)
        self.nb = -(-S // block)
        self.weights = _empty((B, Hkv, S), torch.float32, device)
        self.scores = _empty((B, Hkv, self.nb, self.nb), torch.float32, device)
        self.idx = _empty((B, Hkv, self.nb, topk + n_local), torch.int32, device)
        self.count = _empty((B, Hkv, self.nb), torch.int32, device)
        self.out = _empty((B, Hq, S, D), dtype, device)
        self.lse = _empty((B, Hq, S), torch.float32, device)

    def score(self, v, proj, gain):
        L.dsa_dma_weights(v, proj, gain, self.block, self.weights, self.scores)

    def select(self):
        L.dsa_topk_select(self.scores, self.topk, self.n_local, True, self.idx, self.count)

    def attend(self, q, k, v):
        L.dsa_sparse_attn_prefill_ex(q, k, v, self.idx, self.count, self.block, self.Hq // self.Hkv,
                                     self.weights, self.scale, self.out, self.lse)

    def run(self, q, k, v, proj, gain):
        self.score(v, proj, gain)
        self.select()
        self.attend(q, k, v)
        return self.out


class DecodePlan:
    """Page bounds -> top pages -> attention over the selected pages ([SF] §二-§四)."""

    def __init__(self, B, Hq, Hkv, L_, D, page, topk, dtype, device, scale=None):
        self.B, self.Hq, self.Hkv, self.L, self.D, self.page, self.topk = B, Hq, Hkv, L_, D, page, topk
        self.scale = scale if scale is not None else 1.0 / math.sqrt(D)
        self.nP = L_ // page
        self.kmin = _empty((B, Hkv, self.nP, D), dtype, device)
        self.kmax = _empty((B, Hkv, self.nP, D), dtype, device)
        self.scores = _empty((B, Hkv, 1, self.nP), torch.float32, device)
        self.idx = _empty((B, Hkv, 1, topk), torch.int32, device)
        self.count = _empty((B, Hkv, 1), torch.int32, device)
        ws = L.dsa_sparse_attn_decode_workspace_size(B, Hq, Hkv, topk, page, D)
        self.ws = _empty((ws,), torch.uint8, device)
        self.out = _empty((B, Hq, D), dtype, device)

    def build_metadata(self, k_cache):
        L.dsa_page_minmax(k_cache, self.page, self.kmin, self.kmax)

    def score(self, q):
        L.dsa_block_scores(L.DSA_SCORE_PAGE_BOUND, q, self.kmin, self.kmax, self.page, None,
                           self.scores)

    def select(self):
        L.dsa_topk_select(self.scores, self.topk, 0, False, self.idx, self.count)

    def attend(self, q, k_cache, v_cache):
        L.dsa_sparse_attn_decode(q, k_cache, v_cache, self.idx, self.count, self.page, self.scale,
                                 self.ws, self.out)

    def run(self, q, k_cache, v_cache):
        self.score(q)
        self.select()
        self.attend(q, k_cache, v_cache)
        return self.out


class PagedDecodePlan:
    """Decode over a paged KV pool shared by a batch of sequences of
    different lengths: page bounds through the page table -> top pages ->
    attention over their written tokens ([SF] §二-§四)."""

    def __init__(self, B, Hq, Hkv, D, page, max_pages, topk, device, scale=None):
        self.B, self.Hq, self.Hkv, self.D, self.page = B, Hq, Hkv, D, page
        self.max_pages, self.topk = max_pages, topk
        self.scale = scale if scale is not None else 1.0 / math.sqrt(D)
        self.scores = _empty((B, Hkv, 1, max_pages), torch.float32, device)
        self.idx = _empty((B, Hkv, 1, topk), torch.int32, device)
        self.count = _empty((B, Hkv, 1), torch.int32, device)
        ws = L.dsa_sparse_attn_decode_workspace_size(B, Hq, Hkv, topk, page, D)
        self.ws = _empty((ws,), torch.uint8, device)
        self.out = _empty((B, Hq, D), torch.bfloat16, device)

    def append(self, k_new, v_new, page_table, seq_len, k_pool, v_pool, kmin, kmax):
        L.dsa_paged_append(k_new, v_new, page_table, seq_len, k_pool, v_pool, kmin, kmax)

    def score(self, q, kmin, kmax, page_table, seq_len):
        L.dsa_paged_page_scores(q, kmin, kmax, self.page, page_table, seq_len, self.scores)

    def select(self):
        L.dsa_topk_select(self.scores, self.topk, 0, False, self.idx, self.count)

    def attend(self, q, k_pool, v_pool, page_table, seq_len):
        L.dsa_paged_decode(q, k_pool, v_pool, page_table, seq_len, self.idx, self.count, self.scale,
                           self.ws, self.out)

    def run(self, q, k_pool, v_pool, kmin, kmax, page_table, seq_len):
        self.score(q, kmin, kmax, page_table, seq_len)
        self.select()
        self.attend(q, k_pool, v_pool, page_table, seq_len)
        return self.out


class NSAPlan:
    """Compressed branch (+ block scores) -> top-k blocks -> selected branch;
    sliding branch; gated combine ([NSA] §03)."""

    def __init__(self, B, Hq, Hkv, S, D, cmp_len, cmp_stride, sel_block, sel_k, window, dtype,
                 device, scale=None, per_token=False, fuse_combine=None, fuse_branches=None):
        self.B, self.Hq, self.Hkv, self.S, self.D = B, Hq, Hkv, S, D
        self.cmp_len, self.cmp_stride = cmp_len, cmp_stride
        self.sel_block, self.sel_k, self.window = sel_block, sel_k, window
        self.scale = scale if scale is not None else 1.0 / math.sqrt(D)
        self.n_cmp = (S - cmp_len) // cmp_stride + 1
        self.nb = -(-S // sel_block)
        self.ck = _empty((B, Hkv, self.n_cmp, D), dtype, device)
        self.cv = _empty((B, Hkv, self.n_cmp, D), dtype, device)
        self.o_cmp = _empty((B, Hq, S, D), dtype, device)
        self.lse_cmp = _empty((B, Hq, S), torch.float32, device)
        # per_token: every query token ranks the blocks for its group
        self.per_token = per_token
        # the sliding branch with the gated combine in its epilogue (D = 128,
        # at least 4 query heads per KV head), unless asked otherwise
        self.fuse_combine = (D == 128 and Hq // Hkv >= 4) if fuse_combine is None else fuse_combine
        # the selected and sliding branches and the combine in one pass over
        # each query block's rows (per-block selection, 64k-token blocks);
        # o_sel and o_win are then not written
        eligible = (self.fuse_combine and not per_token and sel_block % 64 == 0
                    and (Hq // Hkv) * sel_block >= 256)
        self.fuse_branches = eligible if fuse_branches is None else (fuse_branches and eligible)
        rows = S if per_token else self.nb
        self.scores = _empty((B, Hkv, rows, self.nb), torch.float32, device)
        self.idx = _empty((B, Hkv, rows, sel_k), torch.int32, device)
        self.count = _empty((B, Hkv, rows), torch.int32, device)
        self.o_sel = _empty((B, Hq, S, D), dtype, device)
        self.o_win = _empty((B, Hq, S, D), dtype, device)
        self.out = _empty((B, Hq, S, D), dtype, device)

    def run(self, q, k, v, z):
        L.dsa_nsa_compress(k, v, self.cmp_len, self.cmp_stride, self.ck, self.cv)
        if self.per_token:
            L.dsa_nsa_cmp_attn(q, self.ck, self.cv, self.cmp_len, self.cmp_stride, self.sel_block,
                               self.scale, self.o_cmp, self.lse_cmp)
            L.dsa_nsa_cmp_token_scores(q, self.ck, self.lse_cmp, self.cmp_len, self.cmp_stride,
                                       self.sel_block, self.scale, self.scores)
            L.dsa_topk_select_tokens(self.scores, self.sel_k, 0, self.sel_block, self.idx,
                                     self.count)
            L.dsa_sparse_attn_tokens(q, k, v, self.idx, self.count, self.sel_block, self.scale,
                                     self.o_sel)
        else:
            L.dsa_nsa_cmp_attn(q, self.ck, self.cv, self.cmp_len, self.cmp_stride,
                               self.sel_block, self.scale, self.o_cmp, self.lse_cmp, self.scores)
            L.dsa_topk_select(self.scores, self.sel_k, 0, True, self.idx, self.count)
            if self.fuse_branches:
                L.dsa_nsa_select_window_combine(q, k, v, self.idx, self.count, self.sel_block,
                                                self.window, self.scale, self.o_cmp, z, self.out)
                return self.out
            L.dsa_sparse_attn_prefill(q, k, v, self.idx, self.count, self.sel_block, 0,
                                      self.scale, self.o_sel)
        if self.fuse_combine:
            L.dsa_nsa_window_combine(q, k, v, self.window, self.scale, self.o_cmp, self.o_sel, z,
                                     self.out)
            return self.out
        L.dsa_sparse_attn_prefill(q, k, v, None, None, self.sel_block, self.window, self.scale,
                                  self.o_win)
        L.dsa_nsa_combine(self.o_cmp, self.o_sel, self.o_win, z, self.out)
        return self.out


class GraphedStep:
    """One step (a zero-argument callable issuing library calls on the current
    stream) captured once into a HIP graph and replayed: the step's launches
    then cost one graph launch.  The library allocates nothing, synchronizes
    nothing and clears no memory with memset inside its calls, so its kernels
    capture as plain kernel nodes.  Inputs and outputs are the tensors the
    callable closes over; refill those in place between replays."""

    def __init__(self, fn, warmup=2):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            fn()

    def __call__(self):
        self.graph.replay()
