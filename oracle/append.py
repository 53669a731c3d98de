"""fp64 decode-step preparation of q, k, v for the paged caches (test
infrastructure only).

The Model Spec page of gemma-4-12b, "Compute-graph nodes", chains three
per-head nodes between ``attn.qkv_proj`` and ``attn.core`` for the new
token of every sequence:

* ``attn.qk_norm`` (``rmsnorm``, eps 1e-6, one weight vector for q and one
  for k, shared by all heads);
* ``attn.v_norm`` (``rmsnormUnit``, eps 1e-6);
* ``attn.rope`` (``rope``) on q and k at the token's position: sliding layers
  theta 10 000, rot = denom = 256, active = 128; global layers theta 10^6,
  rot = denom = 512, active = 64.

On the global layers one 512-wide projection serves as both k and v
("values = keys"); the decode contract of the library stores k only and reads
it as v as well.

The new token of a sequence with ``L`` cached tokens sits at position ``L``
and is written to page ``block_table[b][L // 16]``, slot ``L % 16``.
"""

import numpy as np

from .norm_rope import rmsnorm, rmsnorm_unit, rope

EPS = 1e-6
SLIDING_ROPE = dict(theta=10000.0, rot=256, denom=256, active=128)
GLOBAL_ROPE = dict(theta=1000000.0, rot=512, denom=512, active=64)
PAGE = 16


def decode_step_qkv_sliding(q_raw, k_raw, v_raw, w_q, w_k, positions):
    """q [B,Hq,D], k [B,Hkv,D], v [B,Hkv,D] of the new tokens (fp64)."""
    pos = np.asarray(positions)[:, None]
    q = rope(**SLIDING_ROPE, pos=pos, x=rmsnorm(EPS, q_raw, w_q))
    k = rope(**SLIDING_ROPE, pos=pos, x=rmsnorm(EPS, k_raw, w_k))
    v = rmsnorm_unit(EPS, v_raw)
    return q, k, v


def decode_step_qk_global(q_raw, kv_raw, w_q, w_k, positions):
    """q [B,Hq,D] and the stored k [B,Hkv,D] of the new tokens (fp64)."""
    pos = np.asarray(positions)[:, None]
    q = rope(**GLOBAL_ROPE, pos=pos, x=rmsnorm(EPS, q_raw, w_q))
    k = rope(**GLOBAL_ROPE, pos=pos, x=rmsnorm(EPS, kv_raw, w_k))
    return q, k


def append_targets(block_table, positions):
    """(physical page, slot) where each sequence's new token is stored."""
    bt = np.asarray(block_table)
    pos = np.asarray(positions, dtype=np.int64)
    return bt[np.arange(len(pos)), pos // PAGE], pos % PAGE
