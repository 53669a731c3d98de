"""Checks of the oracle's global decode from the pre-norm projection
(paged_decode_global_prenorm): the cache layout against an independent
scatter, a closed form, an invariance, and its consistency with the sliding
decode oracle over separately built k and v caches. The k / v derivation
itself is pinned against independent references (torch's rms_norm, a
complex rotation with the Model Spec constants, torch attention) in
test_oracle_decode_step.py."""

import numpy as np
import pytest

import oracle
from oracle import paged as P
from workloads import inputs as I


def test_layout_round_trip_and_pair_slots():
    rng = np.random.default_rng(1)
    cache = np.zeros((5, 1, 64, 16, 8), dtype=np.float32)
    bt = np.array([3, 0, 4, 1], dtype=np.int32)
    pos = np.array([0, 5, 17, 40, 63])
    rows = rng.standard_normal((5, 1, 512)).astype(np.float32)
    I.scatter_prenorm(cache, bt, pos, rows)
    np.testing.assert_array_equal(P.gather_prenorm_cache(cache, bt, pos), rows)
    # every chunk is used once per token
    assert sorted(set(P.prenorm_chunk_of(np.arange(0, 512, 8)).tolist())) == list(range(64))
    # the two members of a rotation pair (d, d + 256) sit 16 chunks apart in one half
    d = np.arange(256)
    assert np.all(P.prenorm_chunk_of(d + 256) - P.prenorm_chunk_of(d) == 16)
    assert np.all(P.prenorm_chunk_of(d) // 32 == P.prenorm_chunk_of(d + 256) // 32)


def test_single_key_is_its_unit_norm_row():
    wl = I.make_global_prenorm([1, 1], kv_dtype="f32", tag=(2,))
    got = oracle.paged_decode_global_prenorm(wl.q, wl.x_cache, wl.w_k, wl.block_table, wl.seq_lens, "f32")
    for b in range(2):
        x = P.gather_prenorm_cache(wl.x_cache, wl.block_table[b], [0])[0, 0].astype(np.float64)
        want = x / np.sqrt(np.mean(x * x) + 1e-6)
        np.testing.assert_allclose(got[b], np.broadcast_to(want, (16, 512)), rtol=1e-13, atol=1e-14)


def test_equals_sliding_decode_over_separate_caches():
    # Consistency, not a pin of the k derivation: build row-major k and v
    # caches from the same x (k: weighted norm then RoPE at the token's
    # position, v: unit norm) and run the sliding decode oracle with a window
    # covering every key (full causal decode); the paged gather, the page
    # walk and the attention of the two oracle paths must agree.
    seq_lens = [3, 40, 17]
    wl = I.make_global_prenorm(seq_lens, kv_dtype="bf16", tag=(3,), poison=False)
    got = oracle.paged_decode_global_prenorm(wl.q, wl.x_cache, wl.w_k, wl.block_table, wl.seq_lens, "bf16")
    P_pages = wl.x_cache.shape[0]
    kc = np.zeros((P_pages, 1, 16, 512), dtype=np.float32)
    vc = np.zeros_like(kc)
    for b, L in enumerate(seq_lens):
        pos = np.arange(L)
        x = P.stored_to_f64(P.gather_prenorm_cache(wl.x_cache, wl.block_table[b], pos), "bf16")
        k = oracle.rope(theta=1e6, rot=512, denom=512, active=64, pos=pos[:, None],
                        x=oracle.rmsnorm(1e-6, x, wl.w_k))
        v = oracle.rmsnorm_unit(1e-6, x)
        I.scatter_rowmajor(kc, wl.block_table[b], pos, k.astype(np.float32))
        I.scatter_rowmajor(vc, wl.block_table[b], pos, v.astype(np.float32))
    qf = P.stored_to_f64(wl.q, "bf16").astype(np.float32)
    want = oracle.paged_decode_sliding(qf, kc, vc, wl.block_table, wl.seq_lens, 100, "f32")
    # k and v went through float32 storage above: agreement to fp32 rounding
    np.testing.assert_allclose(got, want, atol=2e-5)


def test_invariant_to_the_scale_of_x():
    wl = I.make_global_prenorm([30, 7], kv_dtype="f32", tag=(4,), poison=False)
    a = oracle.paged_decode_global_prenorm(wl.q, wl.x_cache, wl.w_k, wl.block_table, wl.seq_lens, "f32")
    b = oracle.paged_decode_global_prenorm(wl.q, wl.x_cache * np.float32(8), wl.w_k, wl.block_table,
                                           wl.seq_lens, "f32")
    np.testing.assert_allclose(b, a * 1.0, atol=1e-3)  # only eps breaks the invariance
