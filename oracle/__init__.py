"""Oracle for paged decode attention: plain, slow, fp64 CPU definitions.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
GPU library (``decode_attention_amd``) never imports it, and this package never
imports the library: the two share no code.

Sources (the pages are data; every formula here is restated, not pasted):

* Op Specs page of google/gemma-4-12B, ``Attention.lean``: ``softmax`` (weights
  normalised over the visible positions only), ``causalGQA``, ``slidingGQA``,
  ``decodeGQA`` (the multi-query forms with several consecutive query
  positions per sequence as well).
* Op Specs overview page, "Attention" section and its NOTE on
  ``slidingDecodeGQA`` (decode over the last ``w`` cached positions; no Lean
  definition of its own, semantics from ``slidingGQA``).
* Model Spec page of gemma-4-12b, "Compute-graph nodes" (``attn.core`` rows:
  scale 1, head map h/2 and h/16; ``attn.qk_norm``, ``attn.v_norm`` and
  ``attn.rope`` rows: eps, theta, rot, denom, active) and "Tensors of the
  main nodes" (q, k, v, seq_lens, o shapes).
* Op Specs page, ``Norm.lean`` (``rms``, ``rmsnorm``, ``rmsnormUnit``),
  ``Rope.lean`` (``invFreq``, ``rope``) and ``Attention.lean``
  (``sigmoidGate``); Op Specs overview, "Scalar functions" (``sigmoid``).

Pins: every function here is checked in ``tests/test_oracle_pins.py`` and
``tests/test_oracle_norm_rope.py`` against something other than itself
(literal brute force over the Lean predicates, 50-digit mpmath evaluation,
torch's scaled_dot_product_attention and rms_norm and a rotate-half RoPE from
transformers as library special cases, complex-number rotation, closed forms
and invariants). No function is "parity unpinned".
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
    multiquery_positions,
    paged_multiquery_sliding,
    paged_multiquery_global,
    prenorm_chunk_of,
    gather_prenorm_cache,
    paged_decode_global_prenorm,
    f64_to_bf16_bits,
)
from .norm_rope import (  # noqa: F401
    rms,
    rmsnorm,
    rmsnorm_unit,
    inv_freq,
    rope,
    sigmoid,
    sigmoid_gate,
)
from .append import (  # noqa: F401
    EPS,
    SLIDING_ROPE,
    GLOBAL_ROPE,
    decode_step_qkv_sliding,
    decode_step_qk_global,
    append_targets,
)
