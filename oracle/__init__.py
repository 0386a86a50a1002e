"""fp64 CPU oracle for split-KV paged decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` use it. It shares no code with the
HIP library or its Python binding; the one thing both sides consume is the
seeded input generator (``skvgen``), which holds none of the method.

What it computes (plain definitions, slow on purpose):

* ``decode_attention`` -- for every request, query row and query head: gather
  the visible keys and values through the page table, dequantize them in fp64,
  and evaluate softmax(scale * q.K^T) V as a two-pass softmax, with an optional
  per-head sink logit in the denominator. A row with no visible key is 0.
* ``split_bounds`` / ``split_partials`` / ``combine_flash`` / ``combine_lse`` --
  an fp64 model of the split-KV method itself: per-split statistics
  (m, l, acc), and the two equivalent merges (raw statistics, and normalized
  output plus log-sum-exp). Used to pin the split algebra and to check the
  partial records the GPU path writes.
* ``codecs`` -- storage decoders (bf16 bits, int8 codes, OCP fp8 e4m3fn codes)
  written from the formats' definitions.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
closed forms, library routines and the pages' printed numbers; no function is
"parity unpinned".
"""

from .codecs import decode_bf16_bits, decode_f16_bits, decode_fp8_e4m3fn, decode_storage, fp8_e4m3fn_table
from .attention import (
    SPLIT_ALIGN,
    combine_flash,
    combine_lse,
    decode_attention,
    gather_request,
    row_positions,
    split_bounds,
    split_partials,
    visible_range,
)

__all__ = [
    "SPLIT_ALIGN",
    "combine_flash",
    "combine_lse",
    "decode_attention",
    "decode_bf16_bits",
    "decode_fp8_e4m3fn",
    "decode_storage",
    "decode_f16_bits",
    "fp8_e4m3fn_table",
    "gather_request",
    "row_positions",
    "split_bounds",
    "split_partials",
    "visible_range",
]
