"""Reference oracle for the DeepSeek-V4 hybrid compressed attention step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 CPU
statement of what the GPU path computes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
(the HIP library and its Python binding) never does, and this package imports
nothing from the product.

Sources (web pages; cited by title and section):
  [P1] "DeepSeek-V4, explained" -- the eight-step list of how one query's
       compress-then-select attention layer works, and its glossary.
  [P2] "Decoding DeepSeek-V4" -- section "Compressing the past".
  [P3] "DeepSeek-V4" (visual-learn notes) -- sections "Compress, then select"
       and "A coarse overview alongside local detail".
  [P4] "DeepSeek-V4 Explained: Compressed Sparse Attention and 1M Context at
       10% KV" -- section "The attention stack, and why it is two mechanisms".
  [P5] "DeepSeek-V4: Making a Million Tokens Affordable" -- section
       "Two ways to shrink attention, interleaved".

Modules:
  codecs    OCP FP8 E4M3FN and bfloat16 encode/decode, round-to-nearest-even.
  rope      partial rotary embedding on the last R dims.
  compress  overlapping 2m-window softmax pooling, RMSNorm, RoPE, packing.
  indexer   lightning-indexer scores and the top-k selection rule.
  attend    shared-KV multi-query attention with sink, window, inverse RoPE.

Parity pins live in tests/test_oracle_*.py.  Choices the pages leave open are
fixed by the readings listed at the top of each module.
"""

from . import codecs, rope, compress, indexer, attend  # noqa: F401
