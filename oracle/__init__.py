"""CPU fp64 oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The product path
(the HIP library and its Python binding) never calls it, and the two share
no code: no kernels, headers, helpers, tables or pre/post-processing.

Contents
  dense.attention         full-matrix softmax attention, fp64 (the definition)
  dense.softmax_probs     the normalised probability matrix P of one slice
  dense.attention_rows    the same definition evaluated one output row at a time
  dense.split_partials    per-chunk partial results of split-KV decoding
  dense.merge_partials    the log-sum-exp merge of those partials
  dense.decode_splitkv    split-KV decoding = merge(split(...))
  paged.decode_paged      single-query decoding over a paged KV cache (block tables)
  paged.gather_context    the present context rows of one sequence, in token order
  varlen.attention_varlen attention over a packed batch of variable-length sequences
  backward.attention_backward  dQ, dK, dV of the definition (fp64)
  brute.attention_brute   pure-Python scalar loops, for tiny inputs only
  brute.decode_paged_brute  paged decoding with scalar loops and explicit table lookups
  brute.attention_varlen_brute  packed variable-length attention with scalar loops

Every function is pinned by tests in ``tests/test_oracle.py`` and
``tests/test_oracle_paged.py``, ``tests/test_oracle_varlen.py`` and
``tests/test_oracle_backward.py`` against
closed forms, hand-derived worked examples (``tests/golden/``), invariants of
the definition, brute force and ``torch.nn.functional.scaled_dot_product_attention``
in fp64 on the CPU.  No function here is "parity unpinned".
"""
from .dense import (
    attention,
    attention_rows,
    decode_splitkv,
    merge_partials,
    softmax_probs,
    split_partials,
    split_bounds,
)
from .brute import attention_brute, attention_varlen_brute, decode_paged_brute
from .paged import decode_paged, gather_context
from .varlen import attention_varlen, sequence_bounds
from .backward import attention_backward

__all__ = [
    "attention",
    "attention_rows",
    "decode_splitkv",
    "merge_partials",
    "softmax_probs",
    "split_partials",
    "split_bounds",
    "attention_brute",
    "decode_paged",
    "gather_context",
    "decode_paged_brute",
    "attention_varlen",
    "sequence_bounds",
    "attention_varlen_brute",
    "attention_backward",
]
