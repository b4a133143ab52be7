"""CPU oracle for block-sparse video attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy code that states what the hot path
computes, in float64, for checking the HIP library against.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
library never does, and nothing here imports the library.

Sources (page title, then section):
  * "LVSA: Training-Free Sparse Attention for Long Video Diffusion",
    Meccanismo Core: the frame set A(t) = G u W(t) of a query frame t, the
    rotating periodic global anchors G and the local window W(t), plain or
    expanded to a frame budget C.
  * "Accelerating Text-to-Video Generation with Calibrated Sparse Attention",
    A. Fase di Calibrazione / B. Fase di Inferenza: 128x128 attention blocks,
    a static per-(timestep, layer, head) block mask, attention computed only
    over the selected blocks; the calibration that builds those masks from
    block energies and cross-prompt agreement; spatial repetition (row
    similarity, anchor rows computed and copied).
  * "SQuad: Sub-Quadratic Attention Distillation for Efficient Video
    Generation", 1. Operatore di Attenzione SQuad: the two-pass local/global
    softmax attention.
  * Softmax attention itself (all pages assume full softmax attention inside
    the selected blocks), written as its textbook definition.

Modules:
  masks      frame rule, tile lift, static (SplitMix64) and dense tile masks
  csr        per-query-tile lists of active key tiles
  attention  dense float64 softmax attention with masked blocks set to -inf
  calibration  block energies of dense attention, energy-based block
             selection, cross-prompt aggregation
  squad      two-pass local/global attention (local output as the global
             pass's values)
  repetition spatial-row similarity, repetitive heads, attention on anchor
             rows copied to the other rows, and the inference layer that
             mixes such heads with block-list heads

Every function here is pinned by tests/test_oracle_*.py against values and
properties fixed by the pages or by mathematics (hand-enumerated masks,
brute-force token-level masks, a published SplitMix64 test vector, textbook
full attention, single-block brute force, convex-combination bounds).  The
attention output itself has no printed worked example on the pages; it is
pinned only through those definitions and invariants.
"""
from .masks import (anchor_frames, window_frames, frame_set, frame_mask,
                    expanded_window_frames, frame_set_expanded,
                    frame_mask_expanded, tile_mask_expanded,
                    tile_frame_range, tile_mask_window_anchor,
                    splitmix64_stream, static_hash24, tile_mask_static,
                    tile_mask_dense, tile_mask_block_diagonal, tile_mask)
from .csr import tile_csr
from .calibration import (block_energy, block_energy_rows, select_row,
                          select_mask, aggregate)
from .repetition import (anchor_row, row_cosines, row_cosines_at, repetitive_heads,
                         anchor_count, gather_anchor_rows,
                         broadcast_anchor_rows, repeated_attention,
                         mixed_heads_attention, mixed_heads_attention_rows)
from .squad import (squad_local, squad_attention, squad_attention_rows,
                    window_major_to_position_major,
                    position_major_to_window_major)
from .attention import block_sparse_attention, block_sparse_attention_rows

__all__ = [
    "anchor_frames", "window_frames", "frame_set", "frame_mask",
    "expanded_window_frames", "frame_set_expanded", "frame_mask_expanded",
    "tile_mask_expanded",
    "tile_frame_range", "tile_mask_window_anchor", "splitmix64_stream",
    "static_hash24", "tile_mask_static", "tile_mask_dense", "tile_mask_block_diagonal", "tile_mask",
    "tile_csr", "block_sparse_attention", "block_sparse_attention_rows",
    "block_energy", "block_energy_rows", "select_row", "select_mask",
    "aggregate", "squad_local", "squad_attention", "squad_attention_rows",
    "window_major_to_position_major", "position_major_to_window_major",
    "anchor_row", "row_cosines", "row_cosines_at", "repetitive_heads", "anchor_count",
    "gather_anchor_rows", "broadcast_anchor_rows", "repeated_attention",
    "mixed_heads_attention", "mixed_heads_attention_rows",
]
