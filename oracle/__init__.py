"""Oracle for paged decode attention: plain, slow, fp64 CPU definitions.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
GPU library (``decode_attention_amd``) never imports it, and this package never
imports the library: the two share no code.

Sources (the pages are data; every formula here is restated, not pasted):

* Op Specs page of google/gemma-4-12B, ``Attention.lean``: ``softmax`` (weights
  normalised over the visible positions only), ``causalGQA``, ``slidingGQA``,
  ``decodeGQA``.
* Op Specs overview page, "Attention" section and its NOTE on
  ``slidingDecodeGQA`` (decode over the last ``w`` cached positions; no Lean
  definition of its own, semantics from ``slidingGQA``).
* Model Spec page of gemma-4-12b, "Compute-graph nodes" (``attn.core`` rows:
  scale 1, head map h/2 and h/16) and "Tensors of the main nodes" (q, k, v,
  seq_lens, o shapes).

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
something other than itself (literal brute force over the Lean predicates,
50-digit mpmath evaluation, torch's scaled_dot_product_attention as a library
special case, closed forms and invariants). No function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    softmax_visible,
    causal_gqa,
    sliding_gqa,
    decode_gqa,
    sliding_decode_gqa,
)
from .paged import (  # noqa: F401
    stored_to_f64,
    gather_rowmajor_cache,
    gather_tiled_cache,
    sliding_visible_range,
    paged_decode_sliding,
    paged_decode_global,
)
