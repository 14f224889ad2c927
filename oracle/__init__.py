"""CPU oracle for content-aware block-sparse attention — TEST INFRASTRUCTURE.

A plain, slow, float64 numpy statement of what the library computes.  Only
the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the library itself never does, and this package imports nothing from the
library.  Inputs arrive as numpy arrays (bf16/f32 values upcast exactly to
float64); outputs are float64.

Page key used in citations:
  [DMA]  lsdiaocha.cn/2025/0807/3170092.shtml — retelling of
         "Dynamic Mask Attention" (arXiv:2508.02124).
  [SA]   studyai.ink/2025/08/30 — "什么是稀疏注意力" explainer.
  [NSA]  news.news/tag/稀疏注意力 — summary of "Native Sparse Attention".
  [SF]   techwalker.com/2025/0429/3165971.shtml — retelling of
         "The Sparse Frontier" (arXiv:2504.17768).

Pinning status (the tests under tests/ that check each function against
something other than itself):
  prefill.pool_blocks, prefill.block_scores_pooled   — bilinearity, needles; per-head units
                                                       (sel_heads = 1): pairwise means, heads
                                                       summing to the group score
  prefill.select_blocks                              — brute-force subsets, counts
  prefill.sparse_attention                           — dense causal SDPA, block-diagonal limit,
                                                       softmax invariants, hand worked example;
                                                       per-head lists: explicit per-head dense
                                                       masks from a brute-force top-k, identical
                                                       heads reproducing the group selection
  decode.page_minmax, decode.page_scores             — bound >= true max, equality cases
  decode.decode_attention                            — dense single-query limit
  nsa.compress                                       — stride = len = 1 identity, hand example
  nsa.cmp_attention                                  — dense causal limit (len = stride = 1)
  nsa.cmp_block_scores                               — row-mass invariant and a hand example;
                                                       the overlap-fraction mapping itself is a
                                                       reading, so its split rule is only pinned
                                                       by those two (documented as partly pinned)
  nsa.cmp_token_scores                               — hand example (golden file), row mass = 1,
                                                       block mean = cmp_block_scores
  prefill.select_blocks(row_block)                   — lexsort brute force per token with ties
  nsa.token_sparse_attention                         — dense SDPA with the explicit per-row
                                                       mask; all blocks selected = dense causal
  nsa.window_attention                               — W >= S dense limit, W = 1 identity
  nsa.combine                                        — closed form when branches coincide
  dma.softplus, dma.dynamic_weights                  — softplus identities and limits, v = 0 and
                                                       A = 0 closed forms
  dma.block_weights, dma.block_scores                — hand example, broadcast structure
  dma.biased_sparse_attention                        — dense SDPA with an additive float mask,
                                                       shift invariance under a constant bias
  dma.dma_prefill                                    — planted heavy block selected everywhere
  paged.append, paged.gather                         — appended summaries = min/max of the
                                                       valid tokens; gathered tokens = appended
  paged.page_scores, paged.decode                    — identity table with full pages = the
                                                       contiguous decode oracle; all pages = dense
                                                       SDPA over the valid prefix; -inf past the
                                                       length; invariance under pool permutation
  backward.sparse_attention_backward                 — central finite differences of the
                                                       forward oracle, autograd of a dense masked
                                                       formulation, exact zeros off the mask,
                                                       softmax identities
"""
from . import backward, decode, dma, nsa, paged, prefill  # noqa: F401
