"""Seeded synthetic workloads and the paged KV layouts the kernels read.

This module holds no attention arithmetic. It draws inputs, rounds them to the
storage dtype and writes them into paged caches through block tables. Tests,
``bench.py`` and ``smoke()`` use it to feed both the GPU library and the
oracle.

Input distribution (Model Spec page of gemma-4-12b, "Compute-graph nodes":
``attn.qk_norm`` is a weighted per-head RMSNorm with eps 1e-6,
``attn.v_norm`` an unweighted one, both applied before attention):

* every (token, head) row is x ~ N(0, I_D) (drawn in float32), then
  x_hat = x / sqrt(mean(x^2) + 1e-6);
* q = x_hat * w_q and k = x_hat * w_k, with w_q, w_k ~ N(1, 0.1^2)^D drawn
  once per layer; v = x_hat (unweighted);
* global layers have one cache: values equal keys;
* values are rounded to the storage dtype with round-to-nearest-even (bf16 via
  binary32, so a rare double rounding is possible; the oracle always reads the
  stored values, so this does not affect parity).

Each stream has its own generator ``numpy.random.default_rng([tag, layer,
stream])``: stream 0 seq_lens, 1 block-table permutation, 2 w_q, 3 w_k, 4 q;
the k and v rows of sequence b come from ``[tag, layer, 5, b]`` and
``[tag, layer, 6, b]`` so that sequences can be drawn in parallel threads.

Paged layouts (page = 16 tokens):

* sliding caches: row-major ``[num_pages][Hkv][16][D]``, one for k, one for v;
* global cache: tiled ``[num_pages][Hkv][D/x][16][x]``, x = 16 bytes / element
  size, so 16-byte chunks of x consecutive coordinates are grouped by chunk
  index first and token second.

Block tables are ``int32 [B][P_max]``; entry j of row b is the physical page of
logical page j of sequence b. Logical pages in use are numbered in (b, j)
order and mapped through a seeded permutation of the physical ids. Every other
entry (padding, and sliding pages wholly before the window) points at a guard
page, the last physical page, which is filled with NaN; so are the unused slots
of partly used pages. A kernel that reads outside the visible positions
therefore produces NaN.
"""

import concurrent.futures
import os
from dataclasses import dataclass, field

import numpy as np

PAGE = 16
EPS = 1e-6
BF16_NAN = np.uint16(0x7FC0)

# Gemma-4-12B attention shapes (Model Spec page: "What to watch for" and the
# attn.core rows of "Compute-graph nodes").
SLIDING = dict(Hkv=8, G=2, D=256, window=1024)
GLOBAL = dict(Hkv=1, G=16, D=512)

STREAM_SEQ_LENS, STREAM_PERM, STREAM_WQ, STREAM_WK, STREAM_Q, STREAM_K, STREAM_V = range(7)


def rng_for(tag, layer, stream):
    return np.random.default_rng([int(t) for t in np.atleast_1d(tag)] + [int(layer)]
                                 + [int(s) for s in np.atleast_1d(stream)])


# ----------------------------------------------------------------------------
# storage dtypes
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + r) >> 16).astype(np.uint16)
    return np.where(nan, BF16_NAN, out)


def to_storage(x, kv_dtype):
    """Real rows -> stored array (uint16 bf16 bits, or float32)."""
    if kv_dtype == "bf16":
        return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    if kv_dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(kv_dtype)


def storage_np_dtype(kv_dtype):
    return {"bf16": np.uint16, "f32": np.float32}[kv_dtype]


def storage_nan(kv_dtype):
    return BF16_NAN if kv_dtype == "bf16" else np.float32(np.nan)


def chunk_elems(kv_dtype):
    """x of the tiled layout: elements per 16-byte chunk."""
    return 16 // np.dtype(storage_np_dtype(kv_dtype)).itemsize


# ----------------------------------------------------------------------------
# row generation
# ----------------------------------------------------------------------------

def rms_rows(rng, shape, weight=None):
    """float32 N(0, I) rows (last axis) divided by sqrt(mean(x^2) + 1e-6),
    then multiplied by ``weight`` (one D-vector) if given."""
    x = rng.standard_normal(shape, dtype=np.float32)
    ms = np.einsum("...d,...d->...", x, x) / np.float32(shape[-1])
    x *= (1.0 / np.sqrt(ms + np.float32(EPS)))[..., None]
    if weight is not None:
        x *= np.asarray(weight, dtype=np.float32)
    return x


def _parallel(fn, items, workers=None):
    items = list(items)
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    if workers <= 1 or len(items) <= 1:
        return [fn(i) for i in items]
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


def norm_weight(rng, D):
    return 1.0 + 0.1 * rng.standard_normal(D)


# ----------------------------------------------------------------------------
# layout scatter
# ----------------------------------------------------------------------------

def scatter_rowmajor(cache, bt_row, positions, rows):
    """cache[bt[t // 16], :, t % 16, :] = rows[i] for t = positions[i]."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(bt_row, dtype=np.int64)[positions // PAGE]
    cache[pages, :, positions % PAGE, :] = rows


def scatter_tiled(cache, bt_row, positions, rows):
    """Tiled layout [P][Hkv][D/x][16][x]: element (t, c, d) goes to
    cache[bt[t // 16], c, d // x, t % 16, d % x]."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(bt_row, dtype=np.int64)[positions // PAGE]
    n, hkv, D = rows.shape
    x = cache.shape[-1]
    cache[pages, :, :, positions % PAGE, :] = rows.reshape(n, hkv, D // x, x)


def scatter_prenorm(cache, bt_row, positions, rows):
    """Pre-norm layout [P][Hkv][64][16][8] of 512-wide rows: the 32-coordinate
    block B of a row goes to chunks 32 (B % 2) + 4 (B // 2) .. +4 (so the
    two coordinates d and d + 256 of a rotation pair share a chunk slot in
    the same half), token t to slot t % 16 of page bt[t // 16]."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(bt_row, dtype=np.int64)[positions // PAGE]
    n, hkv, D = rows.shape
    assert D == 512
    blocks = rows.reshape(n, hkv, 16, 4, 8)            # [.., block, chunk in block, 8]
    phys = np.empty((n, hkv, 64, 8), dtype=rows.dtype)
    for B in range(16):
        c0 = 32 * (B % 2) + 4 * (B // 2)
        phys[:, :, c0:c0 + 4, :] = blocks[:, :, B]
    cache[pages, :, :, positions % PAGE, :] = phys


# ----------------------------------------------------------------------------
# block tables
# ----------------------------------------------------------------------------

def build_block_table(page_ranges, P_max, rng):
    """page_ranges[b] = (j_lo, j_hi): logical pages j_lo..j_hi-1 of sequence b
    get physical pages. Returns (block_table int32 [B, P_max], num_pages)
    where the guard page is num_pages - 1."""
    B = len(page_ranges)
    counts = [max(0, hi - lo) for lo, hi in page_ranges]
    n_alloc = int(sum(counts))
    perm = rng.permutation(n_alloc).astype(np.int64)
    guard = n_alloc
    bt = np.full((B, max(int(P_max), 1)), guard, dtype=np.int32)
    k = 0
    for b, (lo, hi) in enumerate(page_ranges):
        if hi > lo:
            bt[b, lo:hi] = perm[k:k + hi - lo]
            k += hi - lo
    return bt, n_alloc + 1


def pages_for(L):
    return (int(L) + PAGE - 1) // PAGE


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclass
class SlidingWorkload:
    q: np.ndarray            # [B, Hkv*G, D] stored
    k_cache: np.ndarray      # [P, Hkv, 16, D] stored
    v_cache: np.ndarray
    block_table: np.ndarray  # int32 [B, P_max]
    seq_lens: np.ndarray     # int32 [B]
    window: int
    kv_dtype: str
    Hkv: int
    G: int
    D: int
    meta: dict = field(default_factory=dict)


@dataclass
class GlobalWorkload:
    q: np.ndarray            # [B, Hkv*G, D] stored
    kv_cache: np.ndarray     # [P, Hkv, D/x, 16, x] stored
    block_table: np.ndarray
    seq_lens: np.ndarray
    kv_dtype: str
    Hkv: int
    G: int
    D: int
    meta: dict = field(default_factory=dict)


def make_sliding(seq_lens, *, Hkv=8, G=2, D=256, window=1024, kv_dtype="bf16",
                 tag=(100,), layer=0, P_max=None, window_only=True,
                 poison=True, q_scale=1.0, q_zero=False):
    """Sliding-layer workload. Only the visible positions [max(0, L-w), L) of
    each sequence are drawn and written; with ``window_only`` only the pages
    that intersect that range are allocated. ``q_scale`` / ``q_zero`` change
    the query distribution for diffuse-softmax test cases."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    if P_max is None:
        P_max = max(1, max((pages_for(L) for L in seq_lens), default=1))
    ranges = []
    for L in seq_lens:
        L = int(L)
        if L <= 0 or window <= 0:
            ranges.append((0, 0))
            continue
        lo = max(0, L - window)
        ranges.append((lo // PAGE if window_only else 0, pages_for(L)))
    bt, num_pages = build_block_table(ranges, P_max, rng_for(tag, layer, STREAM_PERM))
    dt = storage_np_dtype(kv_dtype)
    fill = storage_nan(kv_dtype) if poison else dt(0)
    k_cache = np.full((num_pages, Hkv, PAGE, D), fill, dtype=dt)
    v_cache = np.full((num_pages, Hkv, PAGE, D), fill, dtype=dt)
    w_q = norm_weight(rng_for(tag, layer, STREAM_WQ), D)
    w_k = norm_weight(rng_for(tag, layer, STREAM_WK), D)
    q = rms_rows(rng_for(tag, layer, STREAM_Q), (B, Hkv * G, D), w_q) * np.float32(q_scale)
    if q_zero:
        q = np.zeros_like(q)

    def fill(b):
        L = int(seq_lens[b])
        if L <= 0 or window <= 0:
            return
        pos = np.arange(max(0, L - window), L)
        k = rms_rows(rng_for(tag, layer, [STREAM_K, b]), (len(pos), Hkv, D), w_k)
        scatter_rowmajor(k_cache, bt[b], pos, to_storage(k, kv_dtype))
        v = rms_rows(rng_for(tag, layer, [STREAM_V, b]), (len(pos), Hkv, D))
        scatter_rowmajor(v_cache, bt[b], pos, to_storage(v, kv_dtype))

    _parallel(fill, range(B))
    return SlidingWorkload(to_storage(q, kv_dtype), k_cache, v_cache, bt, seq_lens,
                           int(window), kv_dtype, Hkv, G, D,
                           meta=dict(num_pages=num_pages, P_max=int(bt.shape[1])))


def make_global(seq_lens, *, Hkv=1, G=16, D=512, kv_dtype="bf16", tag=(200,),
                layer=0, P_max=None, poison=True, q_scale=1.0, q_zero=False,
                chunk_tokens=8192):
    """Global-layer workload: one tiled cache (values equal keys)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    if P_max is None:
        P_max = max(1, max((pages_for(L) for L in seq_lens), default=1))
    ranges = [(0, pages_for(L)) if L > 0 else (0, 0) for L in seq_lens]
    bt, num_pages = build_block_table(ranges, P_max, rng_for(tag, layer, STREAM_PERM))
    dt = storage_np_dtype(kv_dtype)
    x = chunk_elems(kv_dtype)
    fill = storage_nan(kv_dtype) if poison else dt(0)
    kv = np.empty((num_pages, Hkv, D // x, PAGE, x), dtype=dt)
    # Fill only what no token overwrites: the guard page and the unused tail
    # slots of each sequence's last page.
    kv[num_pages - 1] = fill
    w_q = norm_weight(rng_for(tag, layer, STREAM_WQ), D)
    w_k = norm_weight(rng_for(tag, layer, STREAM_WK), D)
    q = rms_rows(rng_for(tag, layer, STREAM_Q), (B, Hkv * G, D), w_q) * np.float32(q_scale)
    if q_zero:
        q = np.zeros_like(q)

    def fill_seq(b):
        L = int(seq_lens[b])
        if L <= 0:
            return
        if L % PAGE:
            kv[bt[b, pages_for(L) - 1], :, :, L % PAGE:, :] = fill
        rk = rng_for(tag, layer, [STREAM_K, b])
        for t0 in range(0, L, chunk_tokens):
            pos = np.arange(t0, min(L, t0 + chunk_tokens))
            k = rms_rows(rk, (len(pos), Hkv, D), w_k)
            scatter_tiled(kv, bt[b], pos, to_storage(k, kv_dtype))

    _parallel(fill_seq, range(B))
    return GlobalWorkload(to_storage(q, kv_dtype), kv, bt, seq_lens, kv_dtype, Hkv, G, D,
                          meta=dict(num_pages=num_pages, P_max=int(bt.shape[1])))


@dataclass
class PrenormWorkload:
    q: np.ndarray            # [B, 16, 512] stored (normed and rotated query)
    x_cache: np.ndarray      # pre-norm layout [P, 1, 64, 16, 8] stored
    w_k: np.ndarray          # float32 [512]
    block_table: np.ndarray
    seq_lens: np.ndarray
    kv_dtype: str
    Hkv: int = 1
    G: int = 16
    D: int = 512


def make_global_prenorm(seq_lens, *, kv_dtype="bf16", tag=(950,), layer=0, P_max=None, poison=True,
                        chunk_tokens=8192):
    """Global-layer cache holding the pre-norm kv projection of every token
    (rows N(0, s^2), s log-uniform in [0.1, 10], as raw_rows draws them), the
    k-norm weight, and queries as make_global draws them."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B, Hkv, G, D = len(seq_lens), 1, 16, 512
    if P_max is None:
        P_max = max(1, max((pages_for(L) for L in seq_lens), default=1))
    ranges = [(0, pages_for(L)) if L > 0 else (0, 0) for L in seq_lens]
    bt, num_pages = build_block_table(ranges, P_max, rng_for(tag, layer, STREAM_PERM))
    dt = storage_np_dtype(kv_dtype)
    fill = storage_nan(kv_dtype) if poison else dt(0)
    xc = np.empty((num_pages, Hkv, 64, PAGE, 8), dtype=dt)
    xc[num_pages - 1] = fill
    w_q = norm_weight(rng_for(tag, layer, STREAM_WQ), D)
    w_k = norm_weight(rng_for(tag, layer, STREAM_WK), D).astype(np.float32)
    q = rms_rows(rng_for(tag, layer, STREAM_Q), (B, Hkv * G, D), w_q)

    def fill_seq(b):
        L = int(seq_lens[b])
        if L <= 0:
            return
        if L % PAGE:
            xc[bt[b, pages_for(L) - 1], :, :, L % PAGE:, :] = fill
        rk = rng_for(tag, layer, [STREAM_RAW_K, b])
        for t0 in range(0, L, chunk_tokens):
            pos = np.arange(t0, min(L, t0 + chunk_tokens))
            scatter_prenorm(xc, bt[b], pos, to_storage(raw_rows(rk, (len(pos), Hkv, D)), kv_dtype))

    _parallel(fill_seq, range(B))
    return PrenormWorkload(to_storage(q, kv_dtype), xc, w_k, bt, seq_lens, kv_dtype)


# ----------------------------------------------------------------------------
# several queries per sequence (chunked prefill, speculative verification)
# ----------------------------------------------------------------------------

STREAM_MQ = 12


@dataclass
class MultiQueryWorkload:
    kind: str                # "sliding" or "global"
    q: np.ndarray            # [T, Hkv*G, D] stored; rows q_start[b]..q_start[b+1]-1 are sequence b's
    q_start: np.ndarray      # int32 [B + 1]
    base: object             # the SlidingWorkload / GlobalWorkload holding caches, table and seq_lens

    @property
    def max_queries(self):
        return int(np.max(np.diff(self.q_start), initial=0))


def make_multiquery(kind, seq_lens, q_counts, *, kv_dtype="bf16", tag=(800,), layer=0, P_max=None,
                    q_scale=1.0, **shape):
    """Caches as make_sliding / make_global build them, holding every
    position some query can see, and q_counts[b] queries of sequence b at its
    last q_counts[b] positions. ``shape``: Hkv, G, D (and window for
    sliding)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_counts = np.asarray(q_counts, dtype=np.int32)
    q_start = np.concatenate([[0], np.cumsum(q_counts)]).astype(np.int32)
    if kind == "sliding":
        window = int(shape.pop("window", 1024))
        # the earliest query, S - 1 positions before the last, looks back w - 1
        fill_w = window + max(int(q_counts.max(initial=1)) - 1, 0) if window > 0 else 0
        base = make_sliding(seq_lens, kv_dtype=kv_dtype, tag=tag, layer=layer, P_max=P_max,
                            window=fill_w, **shape)
        base.window = window
    else:
        base = make_global(seq_lens, kv_dtype=kv_dtype, tag=tag, layer=layer, P_max=P_max, **shape)
    Hq = base.Hkv * base.G
    w_q = norm_weight(rng_for(tag, layer, STREAM_WQ), base.D)
    q = rms_rows(rng_for(tag, layer, STREAM_MQ), (int(q_start[-1]), Hq, base.D), w_q) * np.float32(q_scale)
    return MultiQueryWorkload(kind, to_storage(q, kv_dtype), q_start, base)


# ----------------------------------------------------------------------------
# decode-step inputs of the new token (before its norms and rotary embedding)
# ----------------------------------------------------------------------------

STREAM_RAW_Q, STREAM_RAW_K, STREAM_RAW_V, STREAM_FILL = 7, 8, 9, 10


@dataclass
class AppendWorkload:
    kind: str                # "sliding" (separate k/v caches) or "global" (one K=V cache)
    q_raw: np.ndarray        # float32 [B, Hkv*G, D]
    k_raw: np.ndarray        # float32 [B, Hkv, D] (the kv projection on global layers)
    v_raw: object            # float32 [B, Hkv, D], or None on global layers
    w_q: np.ndarray          # float32 [D]
    w_k: np.ndarray          # float32 [D]
    positions: np.ndarray    # int32 [B]
    block_table: np.ndarray  # int32 [B, P_max]
    k_cache: np.ndarray      # stored; sliding [P, Hkv, 16, D], global tiled [P, Hkv, D/x, 16, x]
    v_cache: object          # stored [P, Hkv, 16, D], or None on global layers
    kv_dtype: str
    Hkv: int
    G: int
    D: int


def raw_rows(rng, shape):
    """Pre-norm projection rows: N(0, s^2) with a per-row scale s drawn
    log-uniformly in [0.1, 10] (the norm must undo it)."""
    s = np.exp(rng.uniform(np.log(0.1), np.log(10.0), size=shape[:-1] + (1,)))
    return (rng.standard_normal(shape) * s).astype(np.float32)


STREAM_GATE = 11


def make_gate(shape, tag=(600,), layer=0, scale=2.0):
    """Output-gate logits [B, Hq, D]: float32 N(0, scale^2), so sigmoid(gate)
    spans most of (0, 1)."""
    return (rng_for(tag, layer, STREAM_GATE).standard_normal(shape) * scale).astype(np.float32)


def make_append(kind, positions, *, Hkv, G, D, kv_dtype="bf16", tag=(500,), layer=0,
                P_max=None, block_table=None, k_cache=None, v_cache=None):
    """New-token inputs for ``kind`` ("sliding" or "global") at ``positions``.

    Without caches: every sequence with a valid position gets a page of its
    own for that position, the other block-table entries point at page 0, and
    the caches hold random stored values (so that writes to any other place
    show). With ``block_table`` and caches given (e.g. from make_sliding or
    make_global), those are copied and used as they are."""
    positions = np.asarray(positions, dtype=np.int32)
    B = len(positions)
    sep = kind == "sliding"
    dt = storage_np_dtype(kv_dtype)
    if block_table is None:
        if P_max is None:
            P_max = max(1, int(np.max(positions, initial=0)) // PAGE + 1)
        num_pages = B + 4
        perm = rng_for(tag, layer, STREAM_PERM).permutation(num_pages)
        bt = np.zeros((B, P_max), dtype=np.int32)
        for b, p in enumerate(positions):
            if 0 <= p < P_max * PAGE:
                bt[b, p // PAGE] = perm[b]
        rf = rng_for(tag, layer, STREAM_FILL)
        if sep:
            k_cache = to_storage(rf.standard_normal((num_pages, Hkv, PAGE, D)).astype(np.float32), kv_dtype)
            v_cache = to_storage(rf.standard_normal((num_pages, Hkv, PAGE, D)).astype(np.float32), kv_dtype)
        else:
            x = chunk_elems(kv_dtype)
            k_cache = to_storage(rf.standard_normal((num_pages, Hkv, D // x, PAGE, x)).astype(np.float32), kv_dtype)
            v_cache = None
    else:
        bt = np.array(block_table, dtype=np.int32, copy=True)
        k_cache = np.array(k_cache, dtype=dt, copy=True)
        v_cache = np.array(v_cache, dtype=dt, copy=True) if sep else None
    q_raw = raw_rows(rng_for(tag, layer, STREAM_RAW_Q), (B, Hkv * G, D))
    k_raw = raw_rows(rng_for(tag, layer, STREAM_RAW_K), (B, Hkv, D))
    v_raw = raw_rows(rng_for(tag, layer, STREAM_RAW_V), (B, Hkv, D)) if sep else None
    w_q = norm_weight(rng_for(tag, layer, STREAM_WQ), D).astype(np.float32)
    w_k = norm_weight(rng_for(tag, layer, STREAM_WK), D).astype(np.float32)
    return AppendWorkload(kind, q_raw, k_raw, v_raw, w_q, w_k, positions, bt, k_cache, v_cache,
                          kv_dtype, Hkv, G, D)


# ----------------------------------------------------------------------------
# named configurations (Gemma-4-12B shapes)
# ----------------------------------------------------------------------------

def uniform_seq_lens(tag, B, lo, hi):
    return rng_for(tag, 0, STREAM_SEQ_LENS).integers(lo, hi + 1, size=B).astype(np.int32)


def loguniform_seq_lens(tag, layer, B, L_max):
    u = rng_for(tag, layer, STREAM_SEQ_LENS).random(B)
    return np.maximum(1, np.floor(np.exp(u * np.log(L_max + 1)))).astype(np.int32)


CONFIGS = {
    0: "tiny sliding decode, fp32 KV: B=4, seq_lens {1,17,1024,2048}, Hkv=8, G=2, D=256, window 1024",
    1: "sliding layer decode, bf16 KV, fp32 accumulate: B=64, seq_lens U[1,32768], Hkv=8, G=2, D=256, window 1024",
    2: "global layer decode, bf16 K=V: B=64, seq_lens U[1,32768], Hkv=1, G=16, D=512",
    3: "long-context global decode, bf16 K=V: B=2, seq_lens {131072, 262144}, Hkv=1, G=16, D=512",
}


def config_workload(cfg, layer=0):
    if cfg == 0:
        return make_sliding([1, 17, 1024, 2048], kv_dtype="f32", tag=(0,), layer=layer,
                            P_max=128, **SLIDING)
    if cfg == 1:
        sl = uniform_seq_lens((1,), 64, 1, 32768)
        return make_sliding(sl, kv_dtype="bf16", tag=(1,), layer=layer, P_max=2048, **SLIDING)
    if cfg == 2:
        sl = uniform_seq_lens((2,), 64, 1, 32768)
        return make_global(sl, kv_dtype="bf16", tag=(2,), layer=layer, P_max=2048, **GLOBAL)
    if cfg == 3:
        return make_global([131072, 262144], kv_dtype="bf16", tag=(3,), layer=layer,
                           P_max=16384, **GLOBAL)
    raise ValueError(cfg)


# ----------------------------------------------------------------------------
# the 48-call decode-step sweep, generated on the device
# ----------------------------------------------------------------------------
#
# A full decode step of Gemma-4-12B attends once per layer: 48 layers, layer
# i global iff i % 6 == 5 (8 global, 40 sliding; Model Spec "At a glance"),
# B = 256 sequences with lengths log-uniform in [1, 131072], each layer with
# its own inputs. That is ~66 GB of KV, too much to draw on the host, so the
# caches are drawn on the device with torch's seeded generator (same
# distribution as above: rows N(0, I) rescaled to RMS 1, k times the layer's
# w_k, v unweighted, rounded to bf16 nearest-even); q, the norm weights and
# the block tables are drawn on the host as for the other workloads. Slots no
# query sees (past L in the last page, before the window in the first) and
# the guard page hold NaN. The oracle is fed the stored bytes of sampled
# sequences copied back from the device (sample_to_host).

SWEEP = dict(B=256, L_max=131072, layers=48)
STREAM_DEV_K, STREAM_DEV_V = 20, 21


def sweep_kind(layer):
    return "global" if layer % 6 == 5 else "sliding"


def sweep_seq_lens(tag=(4,), B=SWEEP["B"], L_max=SWEEP["L_max"]):
    """One length draw shared by every layer of the step (the sequences of a batch)."""
    return loguniform_seq_lens(tag, 0, B, L_max)


def torch_seed(tag, layer, stream):
    ss = np.random.SeedSequence([int(t) for t in np.atleast_1d(tag)] + [int(layer), int(stream)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


@dataclass
class DeviceLayer:
    kind: str                  # "sliding" or "global"
    q: object                  # torch bf16 [B, Hq, D]
    caches: tuple              # (k_cache, v_cache) row-major, or (kv_cache,) tiled; torch bf16
    block_table: object        # torch int32 [B, P_max]
    seq_lens: object           # torch int32 [B]
    host_block_table: np.ndarray
    host_seq_lens: np.ndarray
    host_q: np.ndarray         # stored bf16 bits [B, Hq, D]
    window: int
    Hkv: int
    G: int
    D: int


def device_layer(kind, seq_lens, *, tag=(4,), layer=0, window=SLIDING["window"], device="cuda",
                 chunk_pages=8192):
    """One layer of the sweep with its caches drawn on `device`."""
    import torch
    shp = SLIDING if kind == "sliding" else GLOBAL
    Hkv, G, D = shp["Hkv"], shp["G"], shp["D"]
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    P_max = max(1, max(pages_for(L) for L in seq_lens))
    lo_tok = np.maximum(seq_lens.astype(np.int64) - window, 0) if kind == "sliding" else np.zeros(B, np.int64)
    ranges = [((int(lo) // PAGE, pages_for(L)) if L > 0 else (0, 0)) for lo, L in zip(lo_tok, seq_lens)]
    bt, num_pages = build_block_table(ranges, P_max, rng_for(tag, layer, STREAM_PERM))
    counts = np.array([hi - lo for lo, hi in ranges], dtype=np.int64)
    owner = np.repeat(np.arange(B), counts)
    j = np.concatenate([np.arange(lo, hi) for lo, hi in ranges]).astype(np.int64)
    phys = bt[owner, j].astype(np.int64)                    # logical page i -> physical page
    tok = PAGE * j[:, None] + np.arange(PAGE)[None, :]
    visible = (tok >= lo_tok[owner][:, None]) & (tok < seq_lens[owner].astype(np.int64)[:, None])
    n_alloc = len(phys)

    w_q = norm_weight(rng_for(tag, layer, STREAM_WQ), D)
    w_k = norm_weight(rng_for(tag, layer, STREAM_WK), D)
    q_host = to_storage(rms_rows(rng_for(tag, layer, STREAM_Q), (B, Hkv * G, D), w_q), "bf16")
    phys_d = torch.from_numpy(phys).to(device)
    vis_d = torch.from_numpy(visible).to(device)
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device=device)

    def draw(stream, weight):
        if kind == "sliding":
            pool = torch.empty((num_pages, Hkv, PAGE, D), dtype=torch.bfloat16, device=device)
        else:
            pool = torch.empty((num_pages, Hkv, D // 8, PAGE, 8), dtype=torch.bfloat16, device=device)
        pool[num_pages - 1] = float("nan")
        gen = torch.Generator(device=device)
        gen.manual_seed(torch_seed(tag, layer, stream))
        wt = None if weight is None else torch.from_numpy(np.asarray(weight, np.float32)).to(device)
        for c0 in range(0, n_alloc, chunk_pages):
            c1 = min(n_alloc, c0 + chunk_pages)
            x = torch.randn((c1 - c0, PAGE, Hkv, D), generator=gen, device=device, dtype=torch.float32)
            x = x * torch.rsqrt(x.square().mean(-1, keepdim=True) + EPS)
            if wt is not None:
                x = x * wt
            x = torch.where(vis_d[c0:c1, :, None, None], x.to(torch.bfloat16), nan)
            if kind == "sliding":
                page = x.permute(0, 2, 1, 3)                                   # [c, Hkv, 16, D]
            else:
                page = x.reshape(c1 - c0, PAGE, Hkv, D // 8, 8).permute(0, 2, 3, 1, 4)  # [c, Hkv, D/8, 16, 8]
            pool[phys_d[c0:c1]] = page
            del x, page
        return pool

    caches = (draw(STREAM_DEV_K, w_k), draw(STREAM_DEV_V, None)) if kind == "sliding" else (draw(STREAM_DEV_K, w_k),)
    q_dev = torch.from_numpy(q_host.view(np.int16)).to(device).view(torch.bfloat16)
    return DeviceLayer(kind, q_dev, caches, torch.from_numpy(bt).to(device),
                       torch.from_numpy(seq_lens).to(device), bt, seq_lens, q_host, int(window), Hkv, G, D)


def sample_to_host(dl, rows):
    """The stored bytes of sequences `rows` of a DeviceLayer as a host
    workload (compact block table, NaN guard page), for the oracle."""
    import torch
    rows = np.asarray(rows, dtype=np.int64)
    P_max = dl.host_block_table.shape[1]
    picks, table = [], np.zeros((len(rows), P_max), dtype=np.int32)
    n = 0
    for r, b in enumerate(rows):
        L = int(dl.host_seq_lens[b])
        lo = max(0, L - dl.window) // PAGE if dl.kind == "sliding" else 0
        hi = pages_for(L)
        ids = dl.host_block_table[b, lo:hi]
        picks.append(ids)
        table[r, :] = -1
        table[r, lo:hi] = np.arange(n, n + len(ids))
        n += len(ids)
    guard = n
    table[table < 0] = guard
    idx = torch.from_numpy(np.concatenate(picks + [np.array([0])]).astype(np.int64)).to(dl.block_table.device)

    def take(pool):
        got = pool[idx].cpu()
        arr = got.view(torch.int16).numpy().view(np.uint16).copy()
        arr[guard] = BF16_NAN
        return arr

    q = dl.host_q[rows]
    sl = dl.host_seq_lens[rows].astype(np.int32)
    if dl.kind == "sliding":
        return SlidingWorkload(q, take(dl.caches[0]), take(dl.caches[1]), table, sl, dl.window, "bf16",
                               dl.Hkv, dl.G, dl.D)
    return GlobalWorkload(q, take(dl.caches[0]), table, sl, "bf16", dl.Hkv, dl.G, dl.D)
