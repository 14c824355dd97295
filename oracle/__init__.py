"""Plain, slow fp64 CPU oracle for masked attention and its mask representations.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) imports, calls or links anything in this package; only the tests,
the smoke check and the benchmark's CPU-baseline leg do. The oracle shares no code
with the GPU path: no kernels, helpers, tables or pre/post-processing.

Every function states the passage of the source pages it follows. The pages are:

* "opentau.policies.flash_attn_cuda" (API docs): block-id representation,
  ``make_att_block_ids`` and ``flash_attn_blockmask``.
* "tensorplay.nn.attention.varlen": packed layout with cumulative lengths,
  sliding window, GQA; intro: ``seqused_k`` and paged ``block_table``.
* "BinFlash" (README), section "Efficiently Dispatching FlashAttention For
  Partially Filled Attention Masks": coarse block map, 32-bit packed fine mask,
  per-Q-row sorted list of non-empty K blocks, two-pass backward; section "Use":
  (N, N) bool mask, True = attend, default scale 1/sqrt(D).
* "flashinfer.attention.prims_ts.block_sparse_attention": BSR block_indptr /
  block_indices, canonical rows, ``mask_type='causal'`` inside blocks;
  Parameters: ``kv_valid_bits`` and the ``exact_block_bits`` bitmask format.
* "tensorplay.nn.attention.omni_attention", section "Block masks": mask_mod
  predicates, ``and_masks`` / ``or_masks`` / ``noop_mask`` / ``create_mask``;
  intro: ``score_mod`` (the distance-decay bias example); section "Outputs":
  log-sum-exp output.

Pins (what ties each function to something other than itself) live in
``tests/test_oracle_*.py``. Functions without such a pin say "parity unpinned".
"""

from . import masks, attention  # noqa: F401
