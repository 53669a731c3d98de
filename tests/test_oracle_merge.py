"""The split-K log-sum-exp merge, pinned against the oracle's unsplit
decodeGQA ([OS] softmax and decodeGQA).

The global decode splits a sequence's keys into disjoint pieces, keeps per
piece and head the unnormalised output acc_i = sum_l e^(s_l - m_i) v_l, the
reference m_i = max_l s_l and the sum l_i = sum_l e^(s_l - m_i), and merges
  M = max_i m_i,  o = sum_i e^(m_i - M) acc_i / sum_i e^(m_i - M) l_i.
Over the reals this equals the softmax over the union, because the
normaliser is a sum over the visible set. Here the partials are formed in
fp64 from that definition (not from the GPU path), merged, and compared with
the oracle; empty pieces (m = -inf, l = 0) are skipped and the kernels'
base-2 form (scores times log2 e, powers of 2) gives the same result.
"""

import numpy as np
import pytest

import oracle


def _partial(s, v, base2):
    """(acc, m, l) of one piece: s [L'] scores, v [L', D]."""
    if len(s) == 0:
        return np.zeros(v.shape[1]), -np.inf, 0.0
    x = s * (1.0 / np.log(2.0)) if base2 else s
    m = x.max()
    w = np.exp2(x - m) if base2 else np.exp(x - m)
    return w @ v, m, w.sum()


def _merge(parts, base2, rescale=True):
    ms = np.array([p[1] for p in parts])
    if not np.isfinite(ms).any():
        return np.zeros_like(parts[0][0])
    M = ms.max()
    num = np.zeros_like(parts[0][0])
    den = 0.0
    for acc, m, l in parts:
        if m == -np.inf:
            continue
        f = (np.exp2(m - M) if base2 else np.exp(m - M)) if rescale else 1.0
        num += f * acc
        den += f * l
    return num / den


def _cuts(rng, L, n):
    """n pieces of [0, L): sorted cut points, empty pieces allowed."""
    c = np.sort(rng.integers(0, L + 1, size=n - 1))
    return np.concatenate([[0], c, [L]])


def _case(rng, L, D, scale_q):
    q = rng.standard_normal(D) * scale_q
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    return q, k, v


@pytest.mark.parametrize("base2", [False, True])
@pytest.mark.parametrize("L,D,pieces,scale_q", [(1, 4, 1, 1.0), (7, 8, 3, 1.0), (64, 16, 9, 3.0),
                                                  (300, 32, 17, 4.0), (513, 64, 40, 0.0)])
def test_merge_of_pieces_equals_unsplit_decode(base2, L, D, pieces, scale_q):
    rng = np.random.default_rng([L, D, pieces, int(base2)])
    q, k, v = _case(rng, L, D, scale_q)
    # oracle decodeGQA: one KV head, one query head, scale 1, all L keys visible
    ref = oracle.decode_gqa(1.0, q[None, None, :], k[:, None, :], v[:, None, :])[0, 0]
    s = k @ q
    for trial in range(4):
        cuts = _cuts(rng, L, pieces)
        parts = [_partial(s[a:b], v[a:b], base2) for a, b in zip(cuts[:-1], cuts[1:])]
        got = _merge(parts, base2)
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_merge_order_does_not_matter():
    rng = np.random.default_rng(11)
    q, k, v = _case(rng, 200, 16, 3.0)
    s = k @ q
    cuts = _cuts(rng, 200, 12)
    parts = [_partial(s[a:b], v[a:b], True) for a, b in zip(cuts[:-1], cuts[1:])]
    a = _merge(parts, True)
    b = _merge(parts[::-1], True)
    assert np.max(np.abs(a - b)) <= 1e-13


def test_all_pieces_empty_gives_zero():
    parts = [(np.zeros(8), -np.inf, 0.0)] * 3
    assert not _merge(parts, True).any()


def test_planted_merge_without_rescaling_fails():
    # Adding the pieces' numerators and denominators without the
    # e^(m_i - M) factors is wrong as soon as the pieces' maxima differ.
    rng = np.random.default_rng(5)
    q, k, v = _case(rng, 128, 16, 3.0)
    ref = oracle.decode_gqa(1.0, q[None, None, :], k[:, None, :], v[:, None, :])[0, 0]
    s = k @ q
    cuts = np.array([0, 40, 90, 128])
    parts = [_partial(s[a:b], v[a:b], True) for a, b in zip(cuts[:-1], cuts[1:])]
    assert np.max(np.abs(_merge(parts, True) - ref)) <= 1e-12
    assert np.max(np.abs(_merge(parts, True, rescale=False) - ref)) > 1e-3
