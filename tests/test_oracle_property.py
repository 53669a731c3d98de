"""Property-based pin of the fp64 oracle: on random tiny shapes (L <= 40,
D <= 8, Hkv <= 2, G <= 3, S <= 4, every window in [0, L + 2], positions up
to L + 1) the vectorized causalGQA / slidingGQA / decode forms equal a
literal element-by-element evaluation of the Lean definitions
(Attention.lean: softmax, causalGQA, slidingGQA, decodeGQA)."""

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import attention as A
from test_oracle_pins import lean_attention, rand_case

SHAPES = st.tuples(st.integers(1, 4), st.integers(0, 40), st.integers(1, 2), st.integers(1, 3),
                   st.integers(1, 8))


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(shape=SHAPES, seed=st.integers(0, 2**31 - 1), data=st.data())
def test_vectorized_forms_equal_the_definitions(shape, seed, data):
    S, L, Hkv, G, D = shape
    rng = np.random.default_rng(seed)
    q, k, v = rand_case(rng, S, L, Hkv, G, D)
    pos = np.array(data.draw(st.lists(st.integers(0, L + 1), min_size=S, max_size=S)))
    w = data.draw(st.integers(0, L + 2))
    ql, kl, vl = q.tolist(), k.tolist(), v.tolist()
    ref_c = np.array(lean_attention(1.0, pos, ql, kl, vl))
    np.testing.assert_allclose(A.causal_gqa(1.0, pos, q, k, v), ref_c, rtol=1e-12, atol=1e-13)
    ref_s = np.array(lean_attention(1.0, pos, ql, kl, vl, window=w))
    np.testing.assert_allclose(A.sliding_gqa(1.0, w, pos, q, k, v), ref_s, rtol=1e-12, atol=1e-13)
    if L > 0:
        last = [L - 1]
        ref_d = np.array(lean_attention(1.0, last, ql[:1], kl, vl))[0]
        np.testing.assert_allclose(A.decode_gqa(1.0, q[0], k, v), ref_d, rtol=1e-12, atol=1e-13)
        ref_sd = np.array(lean_attention(1.0, last, ql[:1], kl, vl, window=w))[0]
        np.testing.assert_allclose(A.sliding_decode_gqa(1.0, w, q[0], k, v), ref_sd, rtol=1e-12, atol=1e-13)
