"""Float64 CPU oracle for split-KV decode attention (test infrastructure only).

This package is the independent check of the HIP library. Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it; the
library never calls it, and it imports nothing from the library.

What it computes, and where each step comes from:

* ``decode_attention`` -- the plain definition of what Flash-Decoding must
  reproduce: softmax attention of one new query position per sequence over
  its whole cached key/value history (slavadubrov.com, "What is
  Flash-Decoding": "Why decode needs a different schedule" -- the partials are
  reduced into the output that attention over the complete history requires;
  the INT-FlashAttention related-papers page, last abstract: online softmax
  with a running maximum and normalizer gives exact attention). It is the
  unsplit definition, not the split algorithm.
* ``split_partials`` / ``combine_partials`` -- the two steps of the method
  as the same page states them: each split of the history yields a partial
  output plus its log-sum-exp, and a reduction combines them with a correct
  normalization. These exist to check the library's split-only and
  combine-only entry points; their agreement with ``decode_attention`` is
  pinned by brute force in the tests.

Every function is float64 NumPy, one (sequence, kv head) at a time.
"""

from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    decode_values,
    history_rows,
    softmax_attention,
    decode_attention,
    split_length,
    split_partials,
    combine_partials,
)
