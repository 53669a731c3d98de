"""Pins of the fp64 oracle against things other than itself.

* brute force: a literal pure-Python evaluation of the Lean definitions
  (visibility predicates as written, no max subtraction, the denominator
  summed over the filtered positions), on tiny shapes;
* 50-digit mpmath evaluation of the same definitions (fp64 error bound);
* a library special case: torch's scaled_dot_product_attention in float64 on
  the CPU, with an explicit boolean mask, scale 1 and its own GQA head map;
* closed forms: equal logits give the mean of the visible rows, one visible
  key returns its row, two keys give logistic weights (scipy's expit);
* invariants: window >= L reduces sliding to causal, the last row of the
  causal form equals decode, head isolation, convexity, affinity in v, logit
  shift invariance, exactly min(L, w) keys carry weight;
* planted mistakes: mutated copies of the oracle (off-by-one window, wrong
  head map, normalisation over all keys, transposed operand) fail the pins.
"""

import math

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import attention as A


# ----------------------------------------------------------------------------
# literal evaluation of the Lean definitions (Attention.lean)
# ----------------------------------------------------------------------------

def lean_softmax(s, visible, exp=math.exp):
    den = sum(exp(s[m]) for m in range(len(s)) if visible[m])
    return [exp(s[l]) / den if visible[l] else 0 for l in range(len(s))]


def lean_attention(scale, pos, q, k, v, window=None, exp=math.exp, num=float):
    """causalGQA (window None) or slidingGQA, element by element."""
    S, Hkv, G, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    L = len(k)
    Dv = len(v[0][0]) if L else D
    out = [[[[num(0)] * Dv for _ in range(G)] for _ in range(Hkv)] for _ in range(S)]
    for s in range(S):
        for c in range(Hkv):
            for g in range(G):
                logit = [num(scale) * sum(num(q[s][c][g][e]) * num(k[l][c][e]) for e in range(D))
                         for l in range(L)]
                if window is None:
                    vis = [l <= pos[s] for l in range(L)]
                else:
                    vis = [l <= pos[s] and pos[s] < l + window for l in range(L)]
                if not any(vis):
                    continue
                w = lean_softmax(logit, vis, exp)
                for d in range(Dv):
                    out[s][c][g][d] = sum(w[l] * num(v[l][c][d]) for l in range(L))
    return out


def rand_case(rng, S, L, Hkv, G, D, scale_q=0.5):
    q = rng.standard_normal((S, Hkv, G, D)) * scale_q
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    return q, k, v


TINY = [(1, 1, 1, 1, 1), (1, 5, 2, 3, 4), (3, 7, 1, 2, 3), (4, 9, 2, 2, 5), (2, 12, 3, 1, 2)]


@pytest.mark.parametrize("S,L,Hkv,G,D", TINY)
def test_brute_force_causal(S, L, Hkv, G, D):
    rng = np.random.default_rng([1, S, L, Hkv, G, D])
    q, k, v = rand_case(rng, S, L, Hkv, G, D)
    pos = rng.integers(0, L + 2, size=S)
    for scale in (1.0, 0.37):
        ref = np.array(lean_attention(scale, pos, q.tolist(), k.tolist(), v.tolist()))
        got = A.causal_gqa(scale, pos, q, k, v)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("S,L,Hkv,G,D", TINY)
def test_brute_force_sliding_every_window(S, L, Hkv, G, D):
    rng = np.random.default_rng([2, S, L, Hkv, G, D])
    q, k, v = rand_case(rng, S, L, Hkv, G, D)
    pos = rng.integers(0, L + 2, size=S)
    for w in range(0, L + 3):
        ref = np.array(lean_attention(1.0, pos, q.tolist(), k.tolist(), v.tolist(), window=w))
        got = A.sliding_gqa(1.0, w, pos, q, k, v)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("L,Hkv,G,D", [(1, 1, 1, 2), (6, 2, 2, 3), (11, 1, 4, 4)])
def test_brute_force_decode_forms(L, Hkv, G, D):
    rng = np.random.default_rng([3, L, Hkv, G, D])
    q, k, v = rand_case(rng, 1, L, Hkv, G, D)
    ref = np.array(lean_attention(1.0, [L - 1], q.tolist(), k.tolist(), v.tolist()))[0]
    np.testing.assert_allclose(A.decode_gqa(1.0, q[0], k, v), ref, rtol=1e-12, atol=1e-13)
    for w in range(0, L + 3):
        ref = np.array(lean_attention(1.0, [L - 1], q.tolist(), k.tolist(), v.tolist(), window=w))[0]
        np.testing.assert_allclose(A.sliding_decode_gqa(1.0, w, q[0], k, v), ref,
                                   rtol=1e-12, atol=1e-13)


def test_empty_cache_gives_zero():
    q = np.ones((2, 3, 4))
    k = np.zeros((0, 2, 4))
    assert np.all(A.decode_gqa(1.0, q, k, k) == 0)
    assert np.all(A.sliding_decode_gqa(1.0, 5, q, k, k) == 0)


def test_window_zero_gives_zero():
    rng = np.random.default_rng(4)
    q, k, v = rand_case(rng, 1, 9, 2, 2, 3)
    assert np.all(A.sliding_decode_gqa(1.0, 0, q[0], k, v) == 0)


# ----------------------------------------------------------------------------
# 50-digit evaluation: fp64 error bound
# ----------------------------------------------------------------------------

def test_mpmath_50_digits_bounds_fp64_error():
    mpmath.mp.dps = 50
    rng = np.random.default_rng(5)
    # Gemma-like logit scale: rows of RMS 1, D = 24, so logits of several units.
    L, Hkv, G, D = 20, 2, 2, 24
    q, k, v = rand_case(rng, 1, L, Hkv, G, D, scale_q=1.0)
    for w in (None, 7):
        ref = lean_attention(1.0, [L - 1], q.tolist(), k.tolist(), v.tolist(), window=w,
                             exp=mpmath.exp, num=mpmath.mpf)[0]
        got = (A.decode_gqa(1.0, q[0], k, v) if w is None
               else A.sliding_decode_gqa(1.0, w, q[0], k, v))
        for c in range(Hkv):
            for g in range(G):
                for d in range(D):
                    r = ref[c][g][d]
                    err = abs(mpmath.mpf(float(got[c, g, d])) - r)
                    assert err <= mpmath.mpf("1e-13") * max(1, abs(r))


# ----------------------------------------------------------------------------
# library special case: torch SDPA, float64 on the CPU
# ----------------------------------------------------------------------------

def sdpa_reference(scale, visible, q, k, v):
    """q [S, Hkv, G, D] -> torch SDPA with enable_gqa (query head h = c*G + g
    uses key head h // G in torch's own convention)."""
    S, Hkv, G, D = q.shape
    tq = torch.from_numpy(q.reshape(S, Hkv * G, D).transpose(1, 0, 2).copy())[None]
    tk = torch.from_numpy(k.transpose(1, 0, 2).copy())[None]
    tv = torch.from_numpy(v.transpose(1, 0, 2).copy())[None]
    mask = torch.from_numpy(np.asarray(visible, dtype=bool))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                                         enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2).reshape(S, Hkv, G, -1)


def sdpa_error(impl_sliding, seed=6):
    """Max abs difference between impl (slidingGQA signature) and SDPA over
    several shapes, positions and windows (rows with a visible key only)."""
    worst = 0.0
    rng = np.random.default_rng(seed)
    for (S, L, Hkv, G, D) in [(4, 30, 2, 3, 8), (3, 17, 4, 2, 5), (5, 40, 1, 4, 6)]:
        q, k, v = rand_case(rng, S, L, Hkv, G, D, scale_q=1.0)
        pos = rng.integers(0, L, size=S)
        for w in (1, 3, 16, L + 5):
            l = np.arange(L)
            vis = (l[None, :] <= pos[:, None]) & (pos[:, None] < l[None, :] + w)
            ref = sdpa_reference(1.0, vis, q, k, v)
            got = impl_sliding(1.0, w, pos, q, k, v)
            worst = max(worst, float(np.max(np.abs(got - ref))))
    return worst


def test_sdpa_library_pin():
    assert sdpa_error(A.sliding_gqa) < 1e-12


def test_sdpa_library_pin_causal():
    rng = np.random.default_rng(7)
    S, L, Hkv, G, D = 6, 25, 2, 2, 8
    q, k, v = rand_case(rng, S, L, Hkv, G, D, scale_q=1.0)
    pos = rng.integers(0, L, size=S)
    vis = np.arange(L)[None, :] <= pos[:, None]
    np.testing.assert_allclose(A.causal_gqa(1.0, pos, q, k, v),
                               sdpa_reference(1.0, vis, q, k, v), atol=1e-12)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def test_equal_logits_mean_of_visible_rows():
    rng = np.random.default_rng(8)
    L, Hkv, G, D = 13, 2, 2, 5
    _, k, v = rand_case(rng, 1, L, Hkv, G, D)
    q = np.zeros((Hkv, G, D))
    np.testing.assert_allclose(A.decode_gqa(1.0, q, k, v),
                               np.broadcast_to(v.mean(axis=0)[:, None, :], (Hkv, G, D)), atol=1e-14)
    for w in (1, 4, 13, 20):
        n = min(L, w)
        np.testing.assert_allclose(A.sliding_decode_gqa(1.0, w, q, k, v),
                                   np.broadcast_to(v[L - n:].mean(axis=0)[:, None, :], (Hkv, G, D)),
                                   atol=1e-14)


def test_one_visible_key_returns_its_row_exactly():
    rng = np.random.default_rng(9)
    q, k, v = rand_case(rng, 1, 1, 2, 3, 4, scale_q=3.0)
    assert np.array_equal(A.decode_gqa(1.0, q[0], k, v), np.broadcast_to(v[0][:, None, :], (2, 3, 4)))
    q, k, v = rand_case(rng, 1, 9, 2, 3, 4, scale_q=3.0)
    assert np.array_equal(A.sliding_decode_gqa(1.0, 1, q[0], k, v),
                          np.broadcast_to(v[8][:, None, :], (2, 3, 4)))


def test_two_keys_logistic_weights():
    # k rows are orthonormal basis vectors, so the logits are q's coordinates.
    a, b = 1.7, -0.4
    q = np.array([[[a, b, 0.0]]])                  # [Hkv=1, G=1, D=3]
    k = np.array([[[1.0, 0, 0]], [[0, 1.0, 0]]])   # [L=2, 1, 3]
    v = np.array([[[2.0, -1.0, 0.5]], [[-3.0, 4.0, 1.0]]])
    p = scipy.special.expit(a - b)
    expect = p * v[0, 0] + (1 - p) * v[1, 0]
    np.testing.assert_allclose(A.decode_gqa(1.0, q, k, v)[0, 0], expect, rtol=1e-14)
    # scale multiplies the logit difference
    p2 = scipy.special.expit(0.25 * (a - b))
    np.testing.assert_allclose(A.decode_gqa(0.25, q, k, v)[0, 0], p2 * v[0, 0] + (1 - p2) * v[1, 0],
                               rtol=1e-14)


def test_exactly_min_L_w_trailing_keys_carry_weight():
    # v = identity rows: the output row is the weight vector itself.
    L, D = 11, 11
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((L, 1, D))
    v = np.eye(L)[:, None, :]
    for w in range(0, L + 3):
        wts = A.sliding_decode_gqa(1.0, w, q, k, v)[0, 0]
        n = min(L, w)
        assert np.count_nonzero(wts) == n
        assert np.all(wts[:L - n] == 0) and np.all(wts[L - n:] > 0)
        if n:
            assert abs(wts.sum() - 1) < 1e-14


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

def test_window_at_least_L_equals_decode():
    rng = np.random.default_rng(11)
    q, k, v = rand_case(rng, 1, 10, 2, 2, 6)
    full = A.decode_gqa(1.0, q[0], k, v)
    for w in (10, 11, 1000):
        assert np.array_equal(A.sliding_decode_gqa(1.0, w, q[0], k, v), full)


def test_causal_last_row_equals_decode():
    rng = np.random.default_rng(12)
    L = 9
    q, k, v = rand_case(rng, L, L, 2, 2, 4)
    rows = A.causal_gqa(1.0, np.arange(L), q, k, v)
    np.testing.assert_allclose(rows[L - 1], A.decode_gqa(1.0, q[L - 1], k, v), atol=1e-15)
    # and each row s equals decode over the prefix of s + 1 keys
    for s in range(L):
        np.testing.assert_allclose(rows[s], A.decode_gqa(1.0, q[s], k[:s + 1], v[:s + 1]), atol=1e-14)


def test_head_isolation():
    rng = np.random.default_rng(13)
    L, Hkv, G, D = 8, 3, 2, 4
    q, k, v = rand_case(rng, 1, L, Hkv, G, D)
    base = A.decode_gqa(1.0, q[0], k, v)
    k2, v2 = k.copy(), v.copy()
    k2[:, 1] += 5.0
    v2[:, 1] *= -3.0
    pert = A.decode_gqa(1.0, q[0], k2, v2)
    assert np.array_equal(pert[[0, 2]], base[[0, 2]])
    assert not np.allclose(pert[1], base[1])


def test_convexity():
    rng = np.random.default_rng(14)
    L, Hkv, G, D = 30, 2, 2, 6
    q, k, v = rand_case(rng, 1, L, Hkv, G, D, scale_q=2.0)
    for w in (3, 30):
        o = A.sliding_decode_gqa(1.0, w, q[0], k, v)
        vis = v[L - min(L, w):]
        lo = vis.min(axis=0)[:, None, :]
        hi = vis.max(axis=0)[:, None, :]
        assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def test_affine_in_v():
    rng = np.random.default_rng(15)
    q, k, v = rand_case(rng, 1, 12, 2, 2, 5)
    o = A.sliding_decode_gqa(1.0, 7, q[0], k, v)
    np.testing.assert_allclose(A.sliding_decode_gqa(1.0, 7, q[0], k, 2.5 * v - 1.25), 2.5 * o - 1.25,
                               atol=1e-13)


def test_logit_shift_invariance():
    # Append a coordinate where every key holds 1: the logit of every key
    # shifts by the query's value there, which must not change the output.
    rng = np.random.default_rng(16)
    q, k, v = rand_case(rng, 1, 10, 1, 2, 4)
    k1 = np.concatenate([k, np.ones((10, 1, 1))], axis=-1)
    q0 = np.concatenate([q[0], np.zeros((1, 2, 1))], axis=-1)
    q7 = np.concatenate([q[0], np.full((1, 2, 1), 7.0)], axis=-1)
    np.testing.assert_allclose(A.decode_gqa(1.0, q7, k1, v), A.decode_gqa(1.0, q0, k1, v), atol=1e-13)


def test_softmax_weights_sum_to_one_and_match_scipy():
    rng = np.random.default_rng(17)
    s = rng.standard_normal(20) * 4
    vis = rng.random(20) < 0.6
    vis[3] = True
    w = A.softmax_visible(s, vis)
    np.testing.assert_allclose(w[vis], scipy.special.softmax(s[vis]), rtol=1e-14)
    assert np.all(w[~vis] == 0)
    assert A.softmax_visible(s, np.zeros(20, bool)).sum() == 0


# ----------------------------------------------------------------------------
# planted mistakes: each mutant must fail at least one pin
# ----------------------------------------------------------------------------

def mutant_window_off_by_one(scale, window, pos, q, k, v):
    pos = np.asarray(pos)
    l = np.arange(np.asarray(k).shape[0])
    vis = (l[None, :] <= pos[:, None]) & (pos[:, None] <= l[None, :] + window)
    return A._gqa(scale, vis, q, k, v)


def mutant_head_map(scale, window, pos, q, k, v):
    # query head h reads KV head h % Hkv instead of h // G
    S, Hkv, G, D = q.shape
    flat = q.reshape(S, Hkv * G, D)
    perm = np.array([(h % Hkv) * G + (h // Hkv) for h in range(Hkv * G)])
    inv = np.argsort(perm)
    qq = flat[:, perm].reshape(S, Hkv, G, D)
    o = A.sliding_gqa(scale, window, pos, qq, k, v).reshape(S, Hkv * G, -1)
    return o[:, inv].reshape(S, Hkv, G, -1)


def mutant_normalise_over_all(scale, window, pos, q, k, v):
    pos = np.asarray(pos)
    L = np.asarray(k).shape[0]
    l = np.arange(L)
    vis = (l[None, :] <= pos[:, None]) & (pos[:, None] < l[None, :] + window)
    logit = scale * np.einsum("scge,lce->scgl", q, k)
    e = np.exp(logit - logit.max(axis=-1, keepdims=True))
    w = np.where(vis[:, None, None, :], e, 0) / e.sum(axis=-1, keepdims=True)
    return np.einsum("scgl,lcd->scgd", w, v)


def mutant_transposed_operand(scale, window, pos, q, k, v):
    # contracts v over the wrong axis pairing (uses k as values)
    return A.sliding_gqa(scale, window, pos, q, k, k)


@pytest.mark.parametrize("mutant", [mutant_window_off_by_one, mutant_head_map,
                                    mutant_normalise_over_all, mutant_transposed_operand])
def test_planted_mistakes_fail_the_library_pin(mutant):
    assert sdpa_error(mutant) > 1e-3


def test_planted_window_mistake_fails_brute_force():
    rng = np.random.default_rng(18)
    q, k, v = rand_case(rng, 2, 9, 1, 2, 3)
    pos = np.array([8, 5])
    ref = np.array(lean_attention(1.0, pos, q.tolist(), k.tolist(), v.tolist(), window=3))
    assert np.max(np.abs(mutant_window_off_by_one(1.0, 3, pos, q, k, v) - ref)) > 1e-3
