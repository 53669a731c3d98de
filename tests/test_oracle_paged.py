"""Pins of the oracle's paged front end: layout gathers, stored-value decoding,
window range, and the paged wrappers against the logical definitions."""

import numpy as np
import pytest

import oracle
from oracle import attention as A
from oracle import paged as P
from workloads import inputs as I


def test_bf16_decoding_closed_form():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80, 0x4049, 0x0001], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, np.inf, 3.140625, 2.0 ** -133]
    got = P.stored_to_f64(bits, "bf16")
    assert got.dtype == np.float64
    assert list(got) == want


def test_bf16_encoding_round_to_nearest_even():
    x = np.array([1.0 + 2.0 ** -8,            # tie between 1 and 1+2^-7 -> even (1)
                  1.0 + 3 * 2.0 ** -8,        # tie -> even (1 + 2^-6)
                  1.0 + 2.0 ** -8 + 2.0 ** -20,  # above the tie -> up
                  -2.5, np.nan], dtype=np.float32)
    got = I.f32_to_bf16_bits(x)
    assert list(got[:4]) == [0x3F80, 0x3F82, 0x3F81, 0xC020]
    assert np.isnan(P.stored_to_f64(got[4:], "bf16")[0])


def test_sliding_range_matches_predicate_count():
    for L in range(0, 40):
        for w in range(0, 45):
            vis = [l for l in range(L) if l <= L - 1 and L - 1 < l + w]
            lo, hi = P.sliding_visible_range(L, w)
            assert list(range(lo, hi)) == vis


def _brute_gather_rowmajor(cache, bt_row, positions):
    n = len(positions)
    _, hkv, page, D = cache.shape
    out = np.empty((n, hkv, D), dtype=cache.dtype)
    for i, t in enumerate(positions):
        for c in range(hkv):
            for d in range(D):
                out[i, c, d] = cache[bt_row[t // 16], c, t % 16, d]
    return out


def _brute_gather_tiled(cache, bt_row, positions):
    n = len(positions)
    _, hkv, nx, page, x = cache.shape
    out = np.empty((n, hkv, nx * x), dtype=cache.dtype)
    for i, t in enumerate(positions):
        for c in range(hkv):
            for d in range(nx * x):
                out[i, c, d] = cache[bt_row[t // 16], c, d // x, t % 16, d % x]
    return out


def test_gathers_match_elementwise_definition():
    rng = np.random.default_rng(20)
    cache = rng.standard_normal((7, 2, 16, 8)).astype(np.float32)
    bt = rng.permutation(7)
    pos = rng.integers(0, 7 * 16, size=40)
    assert np.array_equal(P.gather_rowmajor_cache(cache, bt, pos), _brute_gather_rowmajor(cache, bt, pos))
    tiled = rng.integers(0, 60000, size=(5, 1, 4, 16, 8)).astype(np.uint16)
    bt = rng.permutation(5)
    pos = rng.integers(0, 5 * 16, size=33)
    assert np.array_equal(P.gather_tiled_cache(tiled, bt, pos), _brute_gather_tiled(tiled, bt, pos))


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_scatter_gather_round_trip(kv_dtype):
    rng = np.random.default_rng(21)
    D, hkv = 16, 2
    x = I.chunk_elems(kv_dtype)
    bt = rng.permutation(6).astype(np.int32)
    rows = I.to_storage(rng.standard_normal((6 * 16, hkv, D)), kv_dtype)
    pos = rng.permutation(6 * 16)
    dt = I.storage_np_dtype(kv_dtype)
    rm = np.zeros((6, hkv, 16, D), dtype=dt)
    I.scatter_rowmajor(rm, bt, pos, rows[pos])
    assert np.array_equal(P.gather_rowmajor_cache(rm, bt, np.arange(96)), rows)
    tl = np.zeros((6, hkv, D // x, 16, x), dtype=dt)
    I.scatter_tiled(tl, bt, pos, rows[pos])
    assert np.array_equal(P.gather_tiled_cache(tl, bt, np.arange(96)), rows)


def _logical_rows(cache_gather, cache, bt_row, L):
    return cache_gather(cache, bt_row, np.arange(L))


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_paged_sliding_equals_logical_definition(kv_dtype):
    # Full (not window-only) allocation without poison, so every position has
    # a finite stored value and the logical slidingDecodeGQA over all L keys
    # (predicate form) can be evaluated directly.
    seq_lens = [1, 5, 16, 17, 40, 63]
    for window in (0, 1, 7, 16, 33, 100):
        wl = I.make_sliding(seq_lens, Hkv=2, G=3, D=8, window=max(window, 1), kv_dtype=kv_dtype,
                            tag=(7, window), window_only=False, poison=False)
        # rows outside the window were never written (zeros); fill all positions
        rng = np.random.default_rng([22, window])
        for b, L in enumerate(seq_lens):
            k = I.to_storage(rng.standard_normal((L, 2, 8)), kv_dtype)
            v = I.to_storage(rng.standard_normal((L, 2, 8)), kv_dtype)
            I.scatter_rowmajor(wl.k_cache, wl.block_table[b], np.arange(L), k)
            I.scatter_rowmajor(wl.v_cache, wl.block_table[b], np.arange(L), v)
        got = P.paged_decode_sliding(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                                     window, kv_dtype)
        qf = P.stored_to_f64(wl.q, kv_dtype)
        for b, L in enumerate(seq_lens):
            k = P.stored_to_f64(_logical_rows(P.gather_rowmajor_cache, wl.k_cache, wl.block_table[b], L), kv_dtype)
            v = P.stored_to_f64(_logical_rows(P.gather_rowmajor_cache, wl.v_cache, wl.block_table[b], L), kv_dtype)
            want = A.sliding_decode_gqa(1.0, window, qf[b].reshape(2, 3, 8), k, v).reshape(6, 8)
            np.testing.assert_allclose(got[b], want, rtol=1e-13, atol=1e-14)


def test_paged_sliding_ignores_poisoned_storage():
    seq_lens = [3, 16, 31, 70]
    a = I.make_sliding(seq_lens, Hkv=2, G=2, D=8, window=20, kv_dtype="bf16", tag=(8,), poison=True)
    b = I.make_sliding(seq_lens, Hkv=2, G=2, D=8, window=20, kv_dtype="bf16", tag=(8,), poison=False)
    oa = P.paged_decode_sliding(a.q, a.k_cache, a.v_cache, a.block_table, a.seq_lens, 20, "bf16")
    ob = P.paged_decode_sliding(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, 20, "bf16")
    assert np.isfinite(oa).all() and np.array_equal(oa, ob)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_paged_global_equals_logical_definition(kv_dtype):
    seq_lens = [1, 15, 16, 17, 50, 0]
    wl = I.make_global(seq_lens, Hkv=1, G=4, D=16, kv_dtype=kv_dtype, tag=(9,))
    got = P.paged_decode_global(wl.q, wl.kv_cache, wl.block_table, wl.seq_lens, kv_dtype)
    qf = P.stored_to_f64(wl.q, kv_dtype)
    for b, L in enumerate(seq_lens):
        if L == 0:
            assert np.all(got[b] == 0)
            continue
        k = P.stored_to_f64(_brute_gather_tiled(wl.kv_cache, wl.block_table[b], np.arange(L)), kv_dtype)
        assert np.isfinite(k).all()
        want = A.decode_gqa(1.0, qf[b].reshape(1, 4, 16), k, k).reshape(4, 16)
        np.testing.assert_allclose(got[b], want, rtol=1e-13, atol=1e-14)


def test_block_table_pages_are_distinct_and_guard_is_poisoned():
    wl = I.make_global([40, 3, 100], Hkv=1, G=2, D=16, kv_dtype="bf16", tag=(10,), P_max=9)
    used = np.concatenate([wl.block_table[b, :I.pages_for(L)] for b, L in enumerate(wl.seq_lens)])
    guard = wl.meta["num_pages"] - 1
    assert len(set(used.tolist())) == len(used) and guard not in used
    assert np.all(wl.block_table[0, 3:] == guard)
    assert np.isnan(P.stored_to_f64(wl.kv_cache[guard], "bf16")).all()


def test_f64_to_bf16_rounding():
    from workloads import inputs as I
    import torch
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.140625, 1.0 + 2**-8 + 2**-40])
    got = oracle.f64_to_bf16_bits(x)
    # exact values stay, midpoints tie to even, and just above a midpoint rounds
    # up (rounding through float32 first would lose the 2^-40 and tie down)
    assert [int(v) for v in got] == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x4049, 0x3F81]
    r = np.random.default_rng(3).standard_normal(100000).astype(np.float32)
    ref_torch = torch.tensor(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(r.astype(np.float64)), ref_torch)
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(r.astype(np.float64)), I.f32_to_bf16_bits(r))


# ---------------------------------------------------------------- several queries per sequence

def test_multiquery_positions():
    np.testing.assert_array_equal(P.multiquery_positions(10, 3), [7, 8, 9])
    np.testing.assert_array_equal(P.multiquery_positions(2, 4), [-2, -1, 0, 1])
    assert len(P.multiquery_positions(5, 0)) == 0


def _truncated_decode(mq, b, s, pos):
    """The decode oracle's output for query row s of sequence b over the same
    caches with the length cut to pos + 1: a causal query at position pos sees
    exactly what the decode query of a pos + 1 token sequence sees."""
    base = mq.base
    q = mq.q[s][None]
    bt = base.block_table[b][None]
    sl = np.array([pos + 1], dtype=np.int32)
    if mq.kind == "sliding":
        return P.paged_decode_sliding(q, base.k_cache, base.v_cache, bt, sl, base.window, base.kv_dtype)[0]
    return P.paged_decode_global(q, base.kv_cache, bt, sl, base.kv_dtype)[0]


@pytest.mark.parametrize("kind", ["sliding", "global"])
def test_multiquery_rows_equal_truncated_decode(kind):
    # Small heads so the decode oracle runs fast; the q counts include 0, 1,
    # more queries than cached tokens, and chunks crossing window and page
    # boundaries.
    shape = dict(Hkv=2, G=2, D=16, window=20) if kind == "sliding" else dict(Hkv=1, G=4, D=32)
    seq_lens = [5, 40, 17, 3, 64, 33]
    counts = [0, 1, 7, 5, 30, 16]
    mq = I.make_multiquery(kind, seq_lens, counts, kv_dtype="bf16", tag=(31, len(kind)), **shape)
    got = (P.paged_multiquery_sliding(mq.q, mq.q_start, mq.base.k_cache, mq.base.v_cache, mq.base.block_table,
                                      mq.base.seq_lens, mq.base.window, "bf16") if kind == "sliding" else
           P.paged_multiquery_global(mq.q, mq.q_start, mq.base.kv_cache, mq.base.block_table, mq.base.seq_lens,
                                     "bf16"))
    assert np.isfinite(got).all()
    for b, (L, S) in enumerate(zip(seq_lens, counts)):
        for j in range(S):
            s, pos = int(mq.q_start[b]) + j, L - S + j  # the last query sits at L - 1
            if pos < 0:
                assert np.all(got[s] == 0)
            else:
                np.testing.assert_allclose(got[s], _truncated_decode(mq, b, s, pos), rtol=1e-12, atol=1e-13)
        if S > 0:  # the last query is the decode query of the untouched sequence
            base = mq.base
            s = int(mq.q_start[b]) + S - 1
            q, bt, sl = mq.q[s][None], base.block_table[b][None], base.seq_lens[b:b + 1]
            ref = (P.paged_decode_sliding(q, base.k_cache, base.v_cache, bt, sl, base.window, "bf16")
                   if kind == "sliding" else P.paged_decode_global(q, base.kv_cache, bt, sl, "bf16"))
            np.testing.assert_allclose(got[s], ref[0], rtol=1e-12, atol=1e-13)


def test_multiquery_sliding_brute_force():
    # Literal per-(query, head, key) loop over the slidingGQA predicate with
    # exp and no max-subtraction, on the gathered logical rows.
    import math
    mq = I.make_multiquery("sliding", [12, 30], [4, 9], kv_dtype="f32", tag=(32,), Hkv=1, G=2, D=4, window=6,
                           q_scale=0.3)
    base = mq.base
    got = P.paged_multiquery_sliding(mq.q, mq.q_start, base.k_cache, base.v_cache, base.block_table,
                                     base.seq_lens, 6, "f32")
    for b, (L, S) in enumerate(zip([12, 30], [4, 9])):
        for j, p in enumerate(range(L - S, L)):
            s = int(mq.q_start[b]) + j
            lo = max(0, p - 5)
            keys = P.gather_rowmajor_cache(base.k_cache, base.block_table[b], np.arange(lo, p + 1)).astype(float)
            vals = P.gather_rowmajor_cache(base.v_cache, base.block_table[b], np.arange(lo, p + 1)).astype(float)
            for h in range(2):
                qv = mq.q[s, h].astype(float)
                e = [math.exp(sum(qv[d] * keys[l, 0, d] for d in range(4))) for l in range(len(keys))]
                z = sum(e)
                for d in range(4):
                    want = sum(e[l] * vals[l, 0, d] for l in range(len(keys))) / z
                    assert abs(got[s, h, d] - want) < 1e-12
