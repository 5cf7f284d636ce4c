"""CPU fp64 oracle for Sparse-VideoGen-style spatio-temporal block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package.  The HIP
library never routes through it, and it shares no code with the HIP path: it
takes the same input *bytes* (from ``svattn_synth``) and recomputes token
coordinates, masks, the token permutation, tile maps and attention on its own,
slowly and plainly.

What it follows ("Accelerating Spatio-Temporal Attention for Video Diffusion on
TPUs", Google for Developers, as retold by three pages):

* dense attention over all query-key pairs, restricted by a mask that keeps only
  some pairs -- aihirek.info, section "A Sparse VideoGen a figyelmi fejeket
  osztályozza", first paragraph;
* spatial heads attend to the query's own and nearby frames, temporal heads to a
  small spatial region across frames -- same section, second paragraph;
* both masks keep full attention to the first frame (the anchor) -- same
  section, third paragraph;
* tiles are empty (skipped), full (no mask needed) or boundary (exact coordinate
  mask needed) -- aihirek.info, section "A TPU-kernel kialakítása döntőnek
  bizonyult", second and third paragraphs;
* temporal heads may run in a temporal-major token order instead of the model's
  frame-major order -- ainews.tenesys.com, list "Co się zmieniło?", item 5.

Readings where the pages are silent (each is listed in the design notes):
  frame-major flattening t = f*P + y*W + x with P = H*W; spatial keep iff
  |f_q - f_k| <= w or f_k == 0; temporal keep iff max(|y_q-y_k|, |x_q-x_k|) <= r
  or f_k == 0 (inclusive windows, clipped at grid edges, anchor on the key side);
  temporal-major order is anchor-first: frame 0 in patch order, then for each
  patch p its frames 1..F-1 (the library's blocked variant lists the patches
  4x4 block by block instead of row by row, its strip variant in snake strips
  two patch columns wide); tile classes count only in-range pairs; masked
  scores are -inf.

Pins (tests/test_oracle_pins.py): closed-form kept counts, the pages' kept
density, hand-worked mask/permutation examples, torch's fp64
scaled_dot_product_attention on the same mask, pure-Python brute force on tiny
inputs, Q = 0 / constant-V closed forms, permute-attend-unpermute equivalence
and an independent geometric derivation of tile classes.
"""
from .core import (  # noqa: F401
    Geometry,
    bf16_to_f64,
    frame_major_coords,
    temporal_major_perm,
    PATCH_BLOCK,
    blocked_patch_order,
    temporal_major_blocked_perm,
    PATCH_STRIP,
    strip_patch_order,
    temporal_major_strips_perm,
    layout_tokens,
    keep_matrix,
    kept_count,
    kept_counts_per_row,
    tile_counts,
    tile_map,
    qtile_order,
    tile_aligned_keep,
    attend_rows,
    attend_head,
    unpermute_rows,
    route_head,
)
