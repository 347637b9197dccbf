"""Float64 CPU oracle for split-KV decode attention (test infrastructure only).

This package is the independent check of the HIP library. Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it; the
library never calls it, and it imports nothing from the library.

What it computes, and where each step comes from:

* ``decode_attention`` -- the plain definition of what Flash-Decoding must
  reproduce: softmax attention of a sequence's single new query over its
  whole cached key/value history (slavadubrov.com, "What is Flash-Decoding":
  "Why decode needs a different schedule" -- merging the split results has
  to give exactly the unsplit attention; the INT-FlashAttention
  related-papers page, last abstract: streaming softmax that tracks the
  running maximum and the running sum is exact, not an approximation). It is
  the unsplit definition, not the split algorithm.
* ``split_partials`` / ``combine_partials`` -- the two steps of the method
  as the same page describes them: every piece of the history gives a
  partial result and its log-sum-exp, and a merge renormalises and adds
  them. These exist to check the library's split-only and
  combine-only entry points; their agreement with ``decode_attention`` is
  pinned by brute force in the tests.

``fp8_e4m3_to_f64`` decodes 8-bit E4M3 cache codes from the format's
definition; ``decode_attention`` with ``kv_dtype="fp8_e4m3"`` and per-kv-head
scales is the definition over the dequantized cache. ``int8_to_f64`` and
``kv_dtype="int8"`` do the same for an 8-bit integer cache, whose scales
``scale_rows`` reads per (position, kv head).

``oracle.sparse`` holds the block-sparse variant (a low-bit key summary,
a top-delta block filter per split, exact attention over the kept blocks),
after the abstract of the "Faster Than Flash" page; its module docstring
lists the readings taken where that page is silent.

Every function is float64 NumPy, one (sequence, kv head) at a time.
"""

from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    fp8_e4m3_to_f64,
    int8_to_f64,
    decode_values,
    history_rows,
    scale_rows,
    softmax_attention,
    decode_attention,
    split_length,
    split_partials,
    combine_partials,
)
from .sparse import (  # noqa: F401
    quantize_block,
    quantize_query,
    log2_units,
    key_summary,
    pack_int4,
    unpack_int4,
    records_to_rows,
    sparse_decode_attention,
)
