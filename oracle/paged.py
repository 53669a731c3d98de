"""Paged-cache front end of the oracle (test infrastructure only).

The pages define the node tensors logically: ``k`` and ``v`` are
[B, S, Hkv, D] with ``seq_lens`` [B] (Model Spec page, "Tensors of the main
nodes", ``attn.core`` row), and the shape domain fixes a page size of 16
("At a glance"). How the cached positions sit in memory is the library's
choice; this module reads the two layouts the library documents, written here
from their definitions:

* row-major paged cache ``[num_pages][Hkv][16][D]`` (sliding layers, separate
  k and v caches): token t of sequence b, KV head c, coordinate d is
  ``cache[bt[b, t // 16], c, t % 16, d]``;
* tiled paged cache ``[num_pages][Hkv][D / x][16][x]`` with x = 16 bytes /
  element size (global layers, one cache read as both k and v): the same
  element is ``cache[bt[b, t // 16], c, d // x, t % 16, d % x]``.

Stored values are decoded exactly to float64 (bf16 bit patterns are the top
16 bits of an IEEE binary32 value).
"""

import numpy as np

from .attention import causal_gqa, decode_gqa, sliding_decode_gqa, sliding_gqa
from .norm_rope import rmsnorm, rmsnorm_unit, rope

PAGE = 16  # tokens per page (Model Spec page, "At a glance", shape domain)


def stored_to_f64(a, kv_dtype):
    """Exact float64 value of stored elements.

    kv_dtype "bf16": ``a`` holds uint16 bit patterns; "f32": ``a`` is float32.
    """
    a = np.asarray(a)
    if kv_dtype == "bf16":
        assert a.dtype == np.uint16
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if kv_dtype == "f32":
        assert a.dtype == np.float32
        return a.astype(np.float64)
    raise ValueError(kv_dtype)


def gather_rowmajor_cache(cache, bt_row, positions):
    """Rows k[t, :, :] ([n, Hkv, D], stored dtype) of a row-major paged cache
    for the logical positions ``positions`` of one sequence."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(bt_row, dtype=np.int64)[positions // PAGE]
    slots = positions % PAGE
    return cache[pages, :, slots, :]


def gather_tiled_cache(cache, bt_row, positions):
    """Rows k[t, :, :] ([n, Hkv, D], stored dtype) of a tiled paged cache
    ``[num_pages][Hkv][D/x][16][x]`` for the logical positions given."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(bt_row, dtype=np.int64)[positions // PAGE]
    slots = positions % PAGE
    sub = cache[pages, :, :, slots, :]          # [n, Hkv, D/x, x]
    n, hkv, nx, x = sub.shape
    return sub.reshape(n, hkv, nx * x)


def prenorm_chunk_of(d):
    """Chunk (of 64 per token) holding coordinate d of a 512-wide pre-norm
    row in the pre-norm cache layout: the 32-coordinate block B = d // 32
    goes to half B % 2, slot B // 2 of that half, and its 4 chunks of 8 in
    order, i.e. chunk 32 * (B % 2) + 4 * (B // 2) + (d % 32) // 8."""
    d = np.asarray(d)
    B = d // 32
    return 32 * (B % 2) + 4 * (B // 2) + (d % 32) // 8


def gather_prenorm_cache(cache, bt_row, positions):
    """Rows x[t, :, :] ([n, Hkv, 512], stored dtype) of a pre-norm paged
    cache ``[num_pages][Hkv][64][16][8]``: coordinate d of token t, KV head c
    is ``cache[bt[t // 16], c, prenorm_chunk_of(d), t % 16, d % 8]``."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(bt_row, dtype=np.int64)[positions // PAGE]
    sub = cache[pages, :, :, positions % PAGE, :]   # [n, Hkv, 64 chunks, 8]
    d = np.arange(512)
    return sub[:, :, prenorm_chunk_of(d), d % 8]


PRENORM_EPS = 1e-6
PRENORM_ROPE = dict(theta=1000000.0, rot=512, denom=512, active=64)


def paged_decode_global_prenorm(q, x_cache, w_k, block_table, seq_lens, kv_dtype, scale=1.0):
    """Global decode from the shared pre-norm projection x (Model Spec page,
    "Compute-graph nodes": on global layers one 512-wide projection feeds
    ``attn.qk_norm`` with ``attn.rope`` as k, and ``attn.v_norm`` as v):
    k[l] = rope(pos l, rmsnorm(eps, x[l], w_k)) with theta 10^6, rot = denom
    = 512, active 64; v[l] = rmsnormUnit(eps, x[l]); then decodeGQA.

    q : [B, Hkv*G, 512] stored (already normed and rotated); x_cache : the
    pre-norm layout; w_k : [512]; returns float64 [B, Hkv*G, 512].
    """
    qf = stored_to_f64(q, kv_dtype)
    B, Hq, D = qf.shape
    Hkv = x_cache.shape[1]
    G = Hq // Hkv
    w = np.asarray(w_k, dtype=np.float64)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        pos = np.arange(L)
        x = stored_to_f64(gather_prenorm_cache(x_cache, block_table[b], pos), kv_dtype)  # [L, Hkv, D]
        k = rope(pos=pos[:, None], x=rmsnorm(PRENORM_EPS, x, w), **PRENORM_ROPE)
        v = rmsnorm_unit(PRENORM_EPS, x)
        out[b] = decode_gqa(scale, qf[b].reshape(Hkv, G, D), k, v).reshape(Hq, D)
    return out


def sliding_visible_range(L, window):
    """Positions visible to the decode query of a sequence of L cached tokens
    under the sliding window: l <= L-1 and L-1 < l + window, i.e. the half-open
    range [max(0, L - window), L) (empty when window = 0 or L = 0)."""
    L = int(L)
    window = int(window)
    if L <= 0 or window <= 0:
        return 0, 0
    return max(0, L - window), L


def paged_decode_sliding(q, k_cache, v_cache, block_table, seq_lens, window,
                         kv_dtype, scale=1.0):
    """Sliding-window decode node (``attn.core`` on sliding layers):
    o[b, h] = sum over the last ``window`` positions of softmax(scale * <q[b,h],
    k[b,s,h // G]>) * v[b,s,h // G].

    q : [B, Hkv*G, D] stored; k_cache, v_cache : row-major paged caches;
    returns float64 [B, Hkv*G, D].

    Only the visible positions are gathered. Every other position has weight
    exactly 0 in the definition, so leaving it out does not change the value;
    it also means storage outside the window is never read (it may hold
    anything, including NaN).
    """
    qf = stored_to_f64(q, kv_dtype)
    B, Hq, D = qf.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        lo, hi = sliding_visible_range(seq_lens[b], window)
        if hi <= lo:
            continue  # nothing visible: the output row stays 0
        pos = np.arange(lo, hi)
        k = stored_to_f64(gather_rowmajor_cache(k_cache, block_table[b], pos), kv_dtype)
        v = stored_to_f64(gather_rowmajor_cache(v_cache, block_table[b], pos), kv_dtype)
        # The gathered keys are the last (hi - lo) <= window positions, so on
        # them slidingDecodeGQA sees every key.
        o = sliding_decode_gqa(scale, window, qf[b].reshape(Hkv, G, D), k, v)
        out[b] = o.reshape(Hq, D)
    return out


def paged_decode_global(q, kv_cache, block_table, seq_lens, kv_dtype, scale=1.0):
    """Global decode node (``attn.core`` on global layers, ``decodeGQA``):
    every cached position is visible and values equal keys, so one tiled cache
    supplies both k and v.

    q : [B, Hkv*G, D] stored; kv_cache : tiled paged cache; returns float64
    [B, Hkv*G, D].
    """
    qf = stored_to_f64(q, kv_dtype)
    B, Hq, D = qf.shape
    Hkv = kv_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        k = stored_to_f64(gather_tiled_cache(kv_cache, block_table[b], np.arange(L)), kv_dtype)
        o = decode_gqa(scale, qf[b].reshape(Hkv, G, D), k, k)
        out[b] = o.reshape(Hq, D)
    return out


def multiquery_positions(L, S):
    """Positions of the S queries of a sequence whose cache holds L tokens,
    the last S of which are the queries' own: query s sits at L - S + s, so
    the last one is at L - 1 (chunked prefill and speculative verification,
    ``causalGQA`` / ``slidingGQA`` with consecutive positions). A negative
    position (S > L) has no cached key at or before it."""
    return int(L) - int(S) + np.arange(int(S), dtype=np.int64)


def _multiquery(q, q_start, seq_lens, kv_dtype, gather, window, scale):
    """Shared front end: per sequence, the queries q[q_start[b]:q_start[b+1]]
    at ``multiquery_positions``; keys gathered from the first position any
    of them can see up to L - 1 (the others have weight exactly 0)."""
    qf = stored_to_f64(q, kv_dtype)
    T, Hq, D = qf.shape
    q_start = np.asarray(q_start, dtype=np.int64)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for b in range(len(seq_lens)):
        t0, t1 = int(q_start[b]), int(q_start[b + 1])
        L, S = int(seq_lens[b]), t1 - t0
        if S <= 0 or L <= 0:
            continue
        pos = multiquery_positions(L, S)
        ok = pos >= 0
        if not ok.any() or (window is not None and window <= 0):
            continue
        lo = 0 if window is None else max(0, int(pos[ok].min()) - int(window) + 1)
        k, v = gather(b, np.arange(lo, L))
        qb = qf[t0:t1][ok]
        Hkv = k.shape[1]
        qb = qb.reshape(len(qb), Hkv, Hq // Hkv, D)
        rel = pos[ok] - lo  # positions within the gathered keys
        if window is None:
            o = causal_gqa(scale, rel, qb, k, v)
        else:
            o = sliding_gqa(scale, window, rel, qb, k, v)
        out[t0:t1][ok] = o.reshape(len(qb), Hq, D)
    return out


def paged_multiquery_sliding(q, q_start, k_cache, v_cache, block_table, seq_lens, window,
                             kv_dtype, scale=1.0):
    """``slidingGQA`` of several queries per sequence over row-major paged
    caches. q : [T, Hkv*G, D] stored, the queries of sequence b in rows
    q_start[b] .. q_start[b+1]-1 at ``multiquery_positions``; returns float64
    [T, Hkv*G, D] (0 for a query that sees no key)."""
    def gather(b, pos):
        k = stored_to_f64(gather_rowmajor_cache(k_cache, block_table[b], pos), kv_dtype)
        v = stored_to_f64(gather_rowmajor_cache(v_cache, block_table[b], pos), kv_dtype)
        return k, v
    return _multiquery(q, q_start, seq_lens, kv_dtype, gather, int(window), scale)


def paged_multiquery_global(q, q_start, kv_cache, block_table, seq_lens, kv_dtype, scale=1.0):
    """``causalGQA`` of several queries per sequence over one tiled paged
    cache read as both k and v (global layers)."""
    def gather(b, pos):
        k = stored_to_f64(gather_tiled_cache(kv_cache, block_table[b], pos), kv_dtype)
        return k, k
    return _multiquery(q, q_start, seq_lens, kv_dtype, gather, None, scale)


def f64_to_bf16_bits(x):
    """bf16 bit patterns of float64 values rounded to nearest, ties to even,
    in one step (no intermediate float32). Domain: finite values within the
    normal bf16 range, as the appended rows are."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    drop = np.uint64(52 - 7)  # fp64 keeps 52 mantissa bits, bf16 keeps 7
    half = np.uint64(1) << (drop - np.uint64(1))
    r = ((bits >> drop) & np.uint64(1)) + half - np.uint64(1)
    rounded = ((bits + r) >> drop) << drop  # the carry moves into the exponent as it should
    y = rounded.view(np.float64).astype(np.float32)  # exact: y has 8 significant bits
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
