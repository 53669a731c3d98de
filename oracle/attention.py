"""fp64 definitions of the attention Op Specs (test infrastructure only).

Each function restates one definition from the Op Specs page of
google/gemma-4-12B (``Attention.lean``) over NumPy float64. Index names follow
the pages: ``s`` query row, ``c`` KV head, ``g`` query head within the group,
``d``/``e`` head-dimension coordinates, ``l`` cached key position.

Shapes (the Lean ``Fin`` arguments, in order):
    q : [S, Hkv, G, D]      k, v : [L, Hkv, D]      result : [S, Hkv, G, D]
"""

import numpy as np


def softmax_visible(s, visible):
    """``softmax s visible`` (Op Specs page of google/gemma-4-12B,
    Attention.lean, ``softmax``).

    The normaliser runs over the visible positions alone: position ``l`` gets
    exp(s_l) / sum over visible m of exp(s_m) when it is visible, else 0. If nothing is visible every weight is 0 (the Lean
    definition never evaluates the denominator then).

    The largest visible logit is subtracted before exponentiating. Numerator
    and denominator are both multiplied by exp(-max), so over the reals the
    value is unchanged; in fp64 it only avoids overflow.

    ``s`` and ``visible`` broadcast against each other; the last axis is l.
    """
    s = np.asarray(s, dtype=np.float64)
    visible = np.broadcast_to(np.asarray(visible, dtype=bool), s.shape)
    masked = np.where(visible, s, -np.inf)
    any_vis = visible.any(axis=-1, keepdims=True)
    m = np.where(any_vis, masked.max(axis=-1, keepdims=True, initial=-np.inf), 0.0)
    e = np.where(visible, np.exp(np.where(visible, s, 0.0) - m), 0.0)
    z = e.sum(axis=-1, keepdims=True)
    return np.where(any_vis, e / np.where(any_vis, z, 1.0), 0.0)


def _gqa(scale, visible, q, k, v):
    """Shared body of causalGQA / slidingGQA: ``visible`` is a [S, L] mask.

    logit[s, c, g, l] = scale * sum_e q[s, c, g, e] * k[l, c, e]
    out[s, c, g, d]   = sum_l softmax(logit, visible[s])[l] * v[l, c, d]
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S, Hkv, G, D = q.shape
    L = k.shape[0]
    assert k.shape == (L, Hkv, D) and v.shape[:2] == (L, Hkv)
    logit = scale * np.einsum("scge,lce->scgl", q, k)
    w = softmax_visible(logit, visible[:, None, None, :])
    return np.einsum("scgl,lcd->scgd", w, v)


def causal_gqa(scale, pos, q, k, v):
    """``causalGQA scale pos q k v``: key l is visible to query s iff
    l <= pos[s]."""
    pos = np.asarray(pos, dtype=np.int64)
    L = np.asarray(k).shape[0]
    l = np.arange(L, dtype=np.int64)
    visible = l[None, :] <= pos[:, None]
    return _gqa(scale, visible, q, k, v)


def sliding_gqa(scale, window, pos, q, k, v):
    """``slidingGQA scale window pos q k v``: with p = pos[s], key l is
    visible to query s iff l <= p and p < l + window, an interval of at most
    ``window`` keys ending at p."""
    pos = np.asarray(pos, dtype=np.int64)
    L = np.asarray(k).shape[0]
    l = np.arange(L, dtype=np.int64)
    p = pos[:, None]
    visible = (l[None, :] <= p) & (p < l[None, :] + int(window))
    return _gqa(scale, visible, q, k, v)


def _last_position(L):
    # Lean's `L - 1` on naturals truncates at 0; with L = 0 there are no keys
    # at all, so the value of pos does not matter.
    return max(int(L) - 1, 0)


def decode_gqa(scale, q, k, v):
    """``decodeGQA scale q k v``: causalGQA with one query placed at L - 1,
    the newest of the L cached positions, so that every key is visible.
    q : [Hkv, G, D]; the KV head of query head c*G+g is c (the index layout
    of q already encodes that)."""
    L = np.asarray(k).shape[0]
    return causal_gqa(scale, [_last_position(L)], np.asarray(q)[None], k, v)[0]


def sliding_decode_gqa(scale, window, q, k, v):
    """``slidingDecodeGQA`` (the graph label of the sliding-window decode node).

    The pages give it no Lean definition; the note on the Op Specs overview
    page describes it as one-query attention restricted to the newest ``w``
    cached positions, windowed as in ``slidingGQA``. Reading taken: slidingGQA with one query at pos = L - 1, so
    the visible keys are L - window < l <= L - 1, i.e. exactly min(L, window)
    keys (none when window = 0).
    """
    L = np.asarray(k).shape[0]
    return sliding_gqa(scale, window, [_last_position(L)], np.asarray(q)[None], k, v)[0]
