"""CPU oracle for MInference-style dynamic sparse attention (TEST INFRASTRUCTURE).

This package is the plain, slow, float64 statement of what the sparse
pre-filling path computes.  It is test infrastructure only: the tests, the
package's smoke check and the benchmark's CPU-baseline leg may import it;
the library and its Python binding never do, and nothing here calls them.
It shares no code with the HIP kernels.

Sources (the pages the method is defined on):
  [P1] "MInference (Milliontokens Inference)" abstract, on the taxoreview
       listing page: three attention shapes in long prompts (A-shape,
       Vertical-Slash, Block-Sparse); one pattern per head chosen offline;
       sparse indices built per prompt at inference; attention computed only
       over those indices.
  [P1-PIT] The PIT abstract fragment on the same page: GPU-friendly tiles and
       sparsity-shaped tiles disagree, which wastes coverage.
  [P2] "MInference 1.0: Accelerating Pre-filling for Long-Context LLMs via
       Dynamic Sparse Attention" summary page: "Summary" (the three stages)
       and "Key points" (Vertical-Slash heads score the last queries against
       every key; Block-Sparse heads mean-pool queries and keys in 64-token
       blocks).

Where the pages leave a step open, the reading taken is stated next to the
function (readings R1..R13 of the design notes):
  R1  A-shape = the first ``sink`` keys plus a causal window of ``window`` keys.
  R2  Vertical-Slash scores use the last 64 rows, scale 1/sqrt(d), and a
      causal softmax over each row's whole causal key set.
  R3  Columns and diagonals are reduced by plain sums of probabilities; the
      diagonal index is o = i - j.
  R4  Top-k ties go to the lower index; selections are returned ascending.
  R5  When k exceeds the candidates (early query blocks), all are taken.
  R6  Block-Sparse ranks the raw dot product of the pooled means.
  R7  Each slash contributes, for a 64-row query block, its exact 64-key span;
      spans that overlap or touch are merged; columns outside every span are
      listed separately.  The mask is that union intersected with causality.
  R8  A row with no key gives out = 0 and lse = -inf.
  R15 Chunked prefill: the results of query blocks q_block0.. are the
      whole-sequence results of those blocks.
  R16 Grid heads keep fixed offsets: 0 .. window-1 and tP-w .. tP+w for the
      T previous frames of P tokens; their index is the Vertical-Slash
      conversion of that slash set.
  R17 A Vertical-Slash head may ask for 32-row query blocks (finer
      granularity against the PIT fragment's coverage waste): R7 with 32 in
      place of 64, so a slash keeps a 32-key span per 32-row block and spans
      merge when they overlap or touch.

Every array is numpy float64 (scores, attention) or int64/int32 (indices).
Inputs arrive as bfloat16 values widened exactly to float64 by the caller.

Pins: every function here is checked in tests/test_oracle.py against
closed forms, brute force on tiny inputs, library routines (numpy's trace,
torch's scaled-dot-product attention) and hand-worked fixtures in
tests/golden/; the per-head dispatch (estimate_head, head_index) is checked
by pushing those fixtures and constructions through it for every pattern.
"""
from .core import (  # noqa: F401
    BM,
    vs_probabilities,
    vs_scores,
    topk,
    bs_pool,
    bs_scores,
    bs_select,
    vs_block_index,
    vs_index,
    bs_block_index,
    bs_index,
    ashape_block_index,
    ashape_index,
    grid_offsets,
    grid_block_index,
    dense_block_index,
    dense_index,
    index_to_csr,
    csr_to_index,
    block_mask,
    attention_block,
    attention_head,
    attention_recall,
    topk_mass,
    estimate_head,
    head_index,
    query_block_rows,
)
