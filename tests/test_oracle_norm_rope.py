"""Pins of the oracle's normalisation, rotary-embedding and output-gate
definitions against things other than themselves: library routines
(torch's rms_norm, a rotate-half RoPE from transformers, scipy's expit),
complex-number rotation, 50-digit mpmath, closed forms and invariants."""

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import norm_rope as NR

EPS = 1e-6


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- rmsnorm

def test_rmsnorm_matches_torch_rms_norm():
    r = rng(1)
    x = r.normal(size=(5, 7, 256)) * r.uniform(0.1, 10, size=(5, 7, 1))
    w = r.normal(1.0, 0.1, size=256)
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (256,), torch.tensor(w), EPS).numpy()
    assert np.max(np.abs(oracle.rmsnorm(EPS, x, w) - ref)) < 1e-13
    ref_unit = torch.nn.functional.rms_norm(torch.tensor(x), (256,), None, EPS).numpy()
    assert np.max(np.abs(oracle.rmsnorm_unit(EPS, x) - ref_unit)) < 1e-13


def test_rmsnorm_constant_rows_closed_form():
    w = rng(2).normal(size=512)
    for c in (0.0, 1e-4, 0.5, -3.0, 1e3):
        x = np.full((1, 512), c)
        np.testing.assert_allclose(oracle.rmsnorm(EPS, x, w)[0], c / np.sqrt(c * c + EPS) * w, rtol=1e-14, atol=0)


def test_rmsnorm_mean_square_and_mpmath():
    x = rng(3).normal(size=(4, 256))
    m = np.mean(x * x, axis=-1)
    y = oracle.rmsnorm_unit(EPS, x)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), m / (m + EPS), rtol=1e-13)
    mpmath.mp.dps = 50
    row = [mpmath.mpf(float(v)) for v in x[0]]
    r = mpmath.sqrt(sum(v * v for v in row) / 256 + mpmath.mpf(EPS))
    exact = [float(v / r) for v in row]
    assert np.max(np.abs(y[0] - exact)) < 1e-15


# ---------------------------------------------------------------- rope

def test_inv_freq_values():
    assert oracle.inv_freq(1e4, 256, 128, 0) == 1.0
    np.testing.assert_allclose(oracle.inv_freq(1e4, 256, 128, 64), 1e4 ** -0.5, rtol=1e-15)
    assert oracle.inv_freq(1e6, 512, 64, 64) == 0.0
    assert oracle.inv_freq(1e6, 512, 64, 255) == 0.0
    mpmath.mp.dps = 50
    for theta, denom, i in ((1e6, 512, 37), (1e4, 256, 127)):
        exact = mpmath.power(mpmath.mpf(theta), -mpmath.mpf(2 * i) / denom)
        np.testing.assert_allclose(oracle.inv_freq(theta, denom, 10**6, i), float(exact), rtol=1e-15)


def complex_rope(theta, rot, denom, active, pos, x):
    """RoPE as a complex multiplication: (x_i + i x_{i+half}) e^{i pos w_i}."""
    half = rot // 2
    w = np.array([theta ** (-2 * i / denom) if i < active else 0.0 for i in range(half)])
    z = x[..., :half] + 1j * x[..., half:2 * half]
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * w)
    out = x.copy()
    out[..., :half], out[..., half:2 * half] = z.real, z.imag
    return out


CONFIGS = [oracle.SLIDING_ROPE, oracle.GLOBAL_ROPE, dict(theta=1e4, rot=64, denom=64, active=32)]


@pytest.mark.parametrize("cfg", CONFIGS)
def test_rope_is_complex_rotation(cfg):
    D = max(cfg["rot"], 256)
    r = rng(4)
    x = r.normal(size=(6, 3, D))
    pos = r.integers(0, 262144, size=(6, 3))
    np.testing.assert_allclose(oracle.rope(pos=pos, x=x, **cfg), complex_rope(pos=pos, x=x, **cfg), atol=1e-12)


@pytest.mark.parametrize("cfg", CONFIGS)
def test_rope_matches_transformers_rotate_half(cfg):
    from transformers.models.gemma.modeling_gemma import apply_rotary_pos_emb
    rot = cfg["rot"]
    D = max(rot, 256)
    r = rng(5)
    x = r.normal(size=(2, 4, 9, D))            # [batch, heads, seq, D]
    pos = r.integers(0, 200000, size=(2, 9))   # [batch, seq]
    ang = pos[..., None] * oracle.inv_freq(cfg["theta"], cfg["denom"], cfg["active"], np.arange(rot // 2))
    emb = np.concatenate([ang, ang], axis=-1)
    cos, sin = torch.tensor(np.cos(emb)), torch.tensor(np.sin(emb))
    xt = torch.tensor(x[..., :rot].copy())     # the library routine rotates the first rot coordinates
    got, _ = apply_rotary_pos_emb(xt, xt, cos, sin)
    ref = oracle.rope(pos=pos[:, None, :], x=x, **cfg)
    assert np.max(np.abs(got.numpy() - ref[..., :rot])) < 1e-12
    np.testing.assert_array_equal(ref[..., rot:], x[..., rot:])


def test_rope_invariants():
    cfg = oracle.GLOBAL_ROPE
    r = rng(6)
    x = r.normal(size=(5, 512))
    # position 0 is the identity
    np.testing.assert_array_equal(oracle.rope(pos=np.zeros(5), x=x, **cfg), x)
    pos = r.integers(0, 262144, size=5)
    y = oracle.rope(pos=pos, x=x, **cfg)
    # each pair keeps its length
    np.testing.assert_allclose(x[:, :256] ** 2 + x[:, 256:] ** 2, y[:, :256] ** 2 + y[:, 256:] ** 2, rtol=1e-12)
    # proportional RoPE: pairs with i >= active are left alone
    np.testing.assert_array_equal(y[:, 64:256], x[:, 64:256])
    np.testing.assert_array_equal(y[:, 256 + 64:], x[:, 256 + 64:])
    # rotations compose: rope(p1) after rope(p2) = rope(p1 + p2)
    p1, p2 = r.integers(0, 10000, size=5), r.integers(0, 10000, size=5)
    np.testing.assert_allclose(oracle.rope(pos=p1, x=oracle.rope(pos=p2, x=x, **cfg), **cfg),
                               oracle.rope(pos=p1 + p2, x=x, **cfg), atol=1e-10)


def test_rope_partial_leaves_the_tail():
    cfg = dict(theta=1e4, rot=64, denom=64, active=32)
    x = rng(7).normal(size=(3, 256))
    y = oracle.rope(pos=np.array([5, 77, 1000]), x=x, **cfg)
    np.testing.assert_array_equal(y[:, 64:], x[:, 64:])


def test_rope_scores_depend_on_relative_position():
    # <rope(q, m), rope(k, n)> is a function of m - n only
    cfg = oracle.SLIDING_ROPE
    r = rng(8)
    q, k = r.normal(size=256), r.normal(size=256)
    def score(m, n):
        return float(oracle.rope(pos=np.array(m), x=q, **cfg) @ oracle.rope(pos=np.array(n), x=k, **cfg))
    for m, n, s in ((10, 3, 100), (1000, 999, 5000), (7, 7, 123)):
        assert abs(score(m, n) - score(m + s, n + s)) < 1e-9


def test_planted_rope_mistakes_fail_the_pins():
    cfg = oracle.SLIDING_ROPE
    x = rng(9).normal(size=(4, 256))
    pos = np.array([1, 10, 100, 1000])
    ref = complex_rope(pos=pos, x=x, **cfg)
    # wrong rotation sense
    wrong = NR.rope(pos=-pos, x=x, **cfg)
    assert np.max(np.abs(wrong - ref)) > 1e-3
    # interleaved pairs (2i, 2i+1) instead of (i, i + half)
    perm = np.concatenate([np.arange(0, 256, 2), np.arange(1, 256, 2)])
    inter = np.empty_like(x)
    inter[:, perm] = NR.rope(pos=pos, x=x[:, perm], **cfg)
    assert np.max(np.abs(inter - ref)) > 1e-3


def test_planted_rmsnorm_mistake_fails_torch():
    x = rng(10).normal(size=(3, 256))
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (256,), None, EPS).numpy()
    summed = x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)  # sum instead of mean
    assert np.max(np.abs(summed - ref)) > 1e-2


# ---------------------------------------------------------------- gate

def test_sigmoid_matches_expit_and_gate_closed_forms():
    g = np.linspace(-50, 50, 1001)
    np.testing.assert_allclose(oracle.sigmoid(g), scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    o = rng(11).normal(size=(3, 512))
    np.testing.assert_array_equal(oracle.sigmoid_gate(o, np.zeros_like(o)), o / 2)
    np.testing.assert_array_equal(oracle.sigmoid_gate(o, np.full_like(o, 1e4)), o)
    np.testing.assert_array_equal(oracle.sigmoid_gate(o, np.full_like(o, -1e4)), 0 * o)


# ---------------------------------------------------------------- decode step

def test_decode_step_composition_and_targets():
    r = rng(12)
    B = 3
    pos = np.array([0, 17, 4095])
    q_raw, k_raw, v_raw = r.normal(size=(B, 16, 256)), r.normal(size=(B, 8, 256)), r.normal(size=(B, 8, 256))
    wq, wk = r.normal(1, 0.1, 256), r.normal(1, 0.1, 256)
    q, k, v = oracle.decode_step_qkv_sliding(q_raw, k_raw, v_raw, wq, wk, pos)
    for b in range(B):
        np.testing.assert_allclose(q[b], complex_rope(pos=pos[b], x=oracle.rmsnorm(EPS, q_raw[b], wq),
                                                      **oracle.SLIDING_ROPE), atol=1e-12)
    np.testing.assert_allclose(v, oracle.rmsnorm_unit(EPS, v_raw))
    for b in range(B):  # (k is pinned against torch rms_norm in test_oracle_decode_step.py)
        np.testing.assert_allclose(k[b], complex_rope(pos=pos[b], x=oracle.rmsnorm(EPS, k_raw[b], wk),
                                                      **oracle.SLIDING_ROPE), atol=1e-12)
    bt = np.arange(3 * 300).reshape(3, 300)[:, ::-1]
    pages, slots = oracle.append_targets(bt, pos)
    assert list(slots) == [0, 1, 15]
    assert list(pages) == [bt[0, 0], bt[1, 1], bt[2, 255]]
