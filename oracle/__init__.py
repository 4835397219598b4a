"""Reference oracle for next-scale (scale-wise) attention — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct CPU implementation of what the
GPU library computes, written in NumPy float64.  It exists to check the HIP
path and nothing else: only the test-suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (``scale_wise_attention_amd``) never imports, calls or falls
back to anything in here, and this package imports nothing from the product.

Sources (web pages on visual-autoregressive next-scale generation):

* "SparVAR: Exploring Sparsity in Visual AutoRegressive Modeling for
  Training-Free Acceleration", abstract: every step attends to all tokens of
  all historical scales; attention sinks; cross-scale locality; an index
  mapping between scales; a sparse pattern of later scales predicted from a
  decision scale; a block-wise sparse kernel.
* "ARVAR: Accelerating Visual Autoregressive Model via Attention Retrospect",
  Background & Motivation (a whole token grid per scale, KV caching,
  FlashAttention), Key Design 2 (gather of the retained positions) and Key
  Design 3, Equations (8)-(9) (nearest base + overwrite scatter); Key
  Design 2 also for the attention-guided choice of the retained positions.
* "LiteVAR: Compressing Visual Autoregressive Modelling with Efficient
  Attention and Quantization", method tags "Attention" and "Softmax", and the
  low-bit quantisation of the data precision.

Modules:

* ``schedule``   -- scale offsets and per-token (scale, row, column).
* ``attention``  -- exact block-causal softmax attention, dense and with a
  tile mask, optional query gather.                      (pinned: see tests)
* ``tile_mask``  -- sink + cross-scale window tile mask by pair enumeration,
  and its CSR form.                                       (pinned: see tests)
* ``scatter``    -- nearest-upsampled base overwritten at retained indices.
                                                          (pinned: see tests)
* ``selection``  -- attention-guided saliency of a small step and the Top-K
  choice of the retained positions on a larger grid.     (pinned: see tests)
* ``dynamic_sparse`` -- per-head tile pattern of a later step predicted from
  the attention mass of a decision scale through index mapping.
                                                          (pinned: see tests)
* ``fp8``        -- e4m3 quantisation of queries and keys with one scale per
  (batch, head).                                          (pinned: see tests)

Every function here is pinned by ``-m "not gpu"`` tests against something other
than itself (brute force, closed forms, invariants, library routines); none is
"parity unpinned".
"""

from .schedule import offsets, token_coords, scale_of_tokens
from .attention import attention
from .tile_mask import tile_mask, mask_to_csr, csr_to_mask
from .scatter import nearest_source_index, scatter_restore
from .selection import saliency, selection_scores, select_positions

__all__ = [
    "offsets",
    "token_coords",
    "scale_of_tokens",
    "attention",
    "tile_mask",
    "mask_to_csr",
    "csr_to_mask",
    "nearest_source_index",
    "scatter_restore",
    "saliency",
    "selection_scores",
    "select_positions",
]
