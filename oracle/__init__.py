"""CPU oracle for masked flash-attention prefill, its gradients, and tree
verify.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, fp64 statement of
what the GPU path computes.  Only the test-suite, the package smoke check and
the benchmark's CPU-baseline leg may import it; the library itself never
does, and nothing here imports the library.

Sources (the web pages this method is taken from):
  [sglang-jax#20]  "feat: support custom mask for flash attention" — custom
                   mask + causal flag on ragged paged attention, the flattened
                   custom-mask layout, the size check and the rule that a
                   sliding window needs the causal kind (code-review comments).
  [aphrodite#1526] "[Attention] feat: support PrefixLM" — prefixlm_mask_mod:
                   bidirectional inside the prefix, causal after it.
  [flashinfer#724] "Custom mask slows down attention." — bit-packed custom
                   masks, tree attention for speculative decoding, the
                   32k x 24k block mask with 50 small triangles.
  [MagiAttention#316] "Feature request: chunk-causal mask type for Flex Flash
                   Attention" — (q_range, k_range, attn_type) lists, the type
                   enum 0..3, CHUNK_CAUSAL and its worked expansion.
  [mlxcel#555]     "feat: add Gemma2 sliding-window (local/global) attention" —
                   window ANDed into the causal mask, even layers local.

Modules:
  masks      dense boolean masks for every mask kind (definitions written out)
  attention  fp64 softmax(Q K^T * scale + mask) V over ragged, paged K/V
  backward   fp64 dQ, dK, dV of the same attention for an upstream dO (whole
             sequences, or sampled rows and keys of one head)
  tiles      per-(q-tile, k-tile) FULL / SKIP / PARTIAL classes and words

Parity pins: every function here is pinned by the tests under tests/ that
are marked "not gpu" (worked examples from the pages, closed forms, textbook
routines and brute force).  Readings the pages leave open (INV_CAUSAL and
BI_CAUSAL semantics, the sliding-window boundary) are pinned only against
their own written definition: parity unpinned for those two points.
"""

from . import masks, attention, backward, tiles  # noqa: F401
