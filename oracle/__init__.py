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

Pins (each against something other than the oracle itself):

* attention definitions and the paged front end: ``tests/test_oracle_pins.py``,
  ``tests/test_oracle_paged.py``, ``tests/test_oracle_merge.py`` (literal
  brute force over the Lean predicates, 50-digit mpmath, torch's
  scaled_dot_product_attention, closed forms and invariants);
* norms, RoPE and the gate: ``tests/test_oracle_norm_rope.py`` (torch's
  rms_norm, transformers' rotate-half RoPE, complex rotation, mpmath, scipy's
  expit);
* the decode-step preparation (``decode_step_qkv_sliding``,
  ``decode_step_qk_global``) and the k / v derivation of
  ``paged_decode_global_prenorm``: ``tests/test_oracle_decode_step.py``,
  against torch's rms_norm, a complex rotation with the Model Spec constants
  typed in the test, and torch attention, with planted mistakes (wrong theta
  or active count, w_q for k, RoPE before the norm, v through the weighted
  norm) that must each fail a pin.

No function is "parity unpinned".
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
