"""Float64 CPU oracle for layer-routed hybrid attention (Flux Attention).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``block_sparse_attention_flux_amd``) and imports nothing from it.

What it computes, and where the pages define it
------------------------------------------------
* ``router``    -- Layer Router: pool the first and last 100 prompt tokens,
  run a small MLP, threshold to a hard 0/1 choice per layer.
  (Flux Attention technical summary on gist.science, section 2
  "Methodology", Layer Router and hard routing at inference; the abstract
  on arXiv 2604.07394 for the per-layer FA/SA choice.)
* ``mask``      -- block mask of the Sparse Attention layers: sink blocks plus
  a causal local window of blocks (the pages name block-sparse attention via
  the Block-Sparse-Attention library on the Qwen3-4B model card, "Sample
  Usage"; the sink+window pattern is a reading of them).
* ``dynmask``   -- a content-aware block mask (mean-pooled coarse attention,
  Top-tau selection); the pages only hint at it (model card slug, "Daily
  Papers" page: Prism and RRAttention abstracts), so the definition is a
  reading of those abstracts.
* ``attention`` -- the plain masked-softmax definition
  ``O = softmax(Q K^T / sqrt(d) + mask) V`` with grouped KV heads, for prefill
  and for one-token decode that reuses the prefill route (technical summary,
  section 2, deployment paragraph); and the soft-routed forward
  ``r FA + (1 - r) SA`` (technical summary, section 2, soft routing).

Everything is float64, written for readability, not speed.  Inputs that the
GPU sees as bf16 are widened exactly to float64 before they get here.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, library routines (torch SDPA in float64,
torch Linear) and invariants; none is "parity unpinned".
"""

from .router import pool_positions, pool_mean, router_mlp, threshold_route, route_requests
from .mask import num_blocks, block_mask, mask_to_csr, mask_row_count, mask_nnz
from .dynmask import (pool_blocks, coarse_logits, block_probs, block_probs_rows, select_row, select_blocks,
                      dynamic_block_mask)
from .attention import (
    allowed_matrix,
    attention_probs,
    attention_prefill,
    attention_prefill_varlen,
    attention_decode,
    attention_prefill_soft,
)

__all__ = [
    "pool_positions", "pool_mean", "router_mlp", "threshold_route", "route_requests",
    "num_blocks", "block_mask", "mask_to_csr", "mask_row_count", "mask_nnz",
    "pool_blocks", "coarse_logits", "block_probs", "block_probs_rows", "select_row", "select_blocks",
    "dynamic_block_mask",
    "allowed_matrix", "attention_probs", "attention_prefill",
    "attention_prefill_varlen", "attention_decode", "attention_prefill_soft",
]
