"""Pins of the oracle's decode-step preparation (decode_step_qkv_sliding,
decode_step_qk_global) and of the k / v derivation inside the pre-norm global
decode (paged_decode_global_prenorm) against references built here without
any oracle code:

* the norms are torch's ``rms_norm`` in float64;
* RoPE is a complex rotation whose constants are typed below from the
  gemma-4-12b Model Spec, "Compute-graph nodes", ``attn.qk_norm``,
  ``attn.v_norm`` and ``attn.rope`` rows of the sliding and global layers
  (eps 1e-6; sliding: theta 10^4, pairs (i, i + 128), exponent -2i/256, all
  128 frequencies; global: theta 10^6, pairs (i, i + 256), exponent -2i/512,
  the first 64 frequencies only);
* attention is torch's ``scaled_dot_product_attention`` in float64 with
  scale 1.

Each plausible mistake listed in ``MUTANTS`` is planted in the oracle (on the
CPU, by replacing one of its constants or one of the helpers it calls) and
must make one of these pins fail.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
from oracle import append as A
from oracle import norm_rope as NR
from oracle import paged as P
from workloads import inputs as I

EPS = 1e-6
# Model Spec constants, typed here (not read from the oracle)
SPEC = {
    "sliding": dict(D=256, theta=1e4, half=128, denom=256, active=128),
    "global": dict(D=512, theta=1e6, half=256, denom=512, active=64),
}
POSITIONS = np.array([0, 1, 15, 16, 1023, 4095, 131071, 262143])


def ref_norm(x, w=None):
    """torch rms_norm over the last axis, float64."""
    t = torch.tensor(np.asarray(x, dtype=np.float64))
    wt = None if w is None else torch.tensor(np.asarray(w, dtype=np.float64))
    return torch.nn.functional.rms_norm(t, (t.shape[-1],), wt, EPS).numpy()


def ref_rope(x, pos, kind):
    """(x_i + i x_{i+half}) * exp(i pos w_i) with the Model Spec's constants."""
    s = SPEC[kind]
    half = s["half"]
    i = np.arange(half, dtype=np.float64)
    w = np.where(i < s["active"], s["theta"] ** (-2.0 * i / s["denom"]), 0.0)
    x = np.asarray(x, dtype=np.float64)
    z = (x[..., :half] + 1j * x[..., half:2 * half]) * np.exp(1j * np.asarray(pos, np.float64)[..., None] * w)
    out = x.copy()
    out[..., :half], out[..., half:2 * half] = z.real, z.imag
    return out


def raw(seed, shape):
    return I.raw_rows(np.random.default_rng(seed), shape).astype(np.float64)


def weights(seed, D):
    r = np.random.default_rng(seed)
    return r.normal(1.0, 0.1, D), r.normal(1.0, 0.1, D)


# ---------------------------------------------------------------- pin errors
# Each returns the largest deviation of the oracle from the reference; the
# pins assert it is at rounding level, the mutant test that it is not.

def err_step_global():
    B = len(POSITIONS)
    q_raw, kv_raw = raw(1, (B, 16, 512)), raw(2, (B, 1, 512))
    w_q, w_k = weights(3, 512)
    q, k = oracle.decode_step_qk_global(q_raw, kv_raw, w_q, w_k, POSITIONS)
    pos = POSITIONS[:, None]
    eq = np.max(np.abs(q - ref_rope(ref_norm(q_raw, w_q), pos, "global")))
    ek = np.max(np.abs(k - ref_rope(ref_norm(kv_raw, w_k), pos, "global")))
    return max(eq, ek)


def err_step_sliding():
    B = len(POSITIONS)
    q_raw, k_raw, v_raw = raw(4, (B, 16, 256)), raw(5, (B, 8, 256)), raw(6, (B, 8, 256))
    w_q, w_k = weights(7, 256)
    q, k, v = oracle.decode_step_qkv_sliding(q_raw, k_raw, v_raw, w_q, w_k, POSITIONS)
    pos = POSITIONS[:, None]
    eq = np.max(np.abs(q - ref_rope(ref_norm(q_raw, w_q), pos, "sliding")))
    ek = np.max(np.abs(k - ref_rope(ref_norm(k_raw, w_k), pos, "sliding")))
    ev = np.max(np.abs(v - ref_norm(v_raw)))
    return max(eq, ek, ev)


@functools.lru_cache(maxsize=None)
def prenorm_case(seq_lens=(1, 5, 40, 300), start=(0, 0, 100, 3000), seed=8):
    """Pre-norm rows x of every token, scattered into an fp32 pre-norm cache
    at logical positions start[b] .. start[b] + L - 1 (the decode of a
    sequence sees positions 0 .. L - 1, so ``start`` > 0 shifts the cached
    tokens into far pages by giving the sequence a longer length)."""
    r = np.random.default_rng(seed)
    lens = [s + L for s, L in zip(start, seq_lens)]
    P_max = max(I.pages_for(L) for L in lens)
    n_pages = sum(I.pages_for(L) for L in lens)
    perm = r.permutation(n_pages)
    bt = np.zeros((len(lens), P_max), dtype=np.int32)
    cache = np.zeros((n_pages, 1, 64, 16, 8), dtype=np.float32)
    xs, k0 = [], 0
    for b, L in enumerate(lens):
        npg = I.pages_for(L)
        bt[b, :npg] = perm[k0:k0 + npg]
        k0 += npg
        x = I.raw_rows(r, (L, 1, 512))
        I.scatter_prenorm(cache, bt[b], np.arange(L), x)
        xs.append(x.astype(np.float64))
    q = I.rms_rows(r, (len(lens), 16, 512)).astype(np.float32)
    w_k = (1.0 + 0.1 * r.standard_normal(512)).astype(np.float32)
    return q, cache, w_k, bt, np.array(lens, dtype=np.int32), xs


def ref_prenorm_decode(q, xs, w_k):
    out = np.zeros(q.shape, dtype=np.float64)
    for b, x in enumerate(xs):
        L = len(x)
        k = ref_rope(ref_norm(x[:, 0], w_k), np.arange(L), "global")      # [L, 512]
        v = ref_norm(x[:, 0])
        qt = torch.tensor(q[b].astype(np.float64))[None, :, None, :]       # [1, 16, 1, 512]
        kt = torch.tensor(k)[None, None].expand(1, 16, L, 512)
        vt = torch.tensor(v)[None, None].expand(1, 16, L, 512)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=1.0)
        out[b] = o[0, :, 0, :].numpy()
    return out


def err_prenorm():
    q, cache, w_k, bt, lens, xs = prenorm_case()
    got = oracle.paged_decode_global_prenorm(q, cache, w_k, bt, lens, "f32")
    return np.max(np.abs(got - ref_prenorm_decode(q, xs, w_k)))


# ---------------------------------------------------------------- the pins

def test_decode_step_global_q_and_k():
    assert err_step_global() < 1e-11


def test_decode_step_sliding_q_k_v():
    assert err_step_sliding() < 1e-11


def test_position_zero_is_the_weighted_norm():
    # RoPE at position 0 is the identity, on both layer kinds
    q_raw, kv_raw = raw(9, (2, 16, 512)), raw(10, (2, 1, 512))
    w_q, w_k = weights(11, 512)
    q, k = oracle.decode_step_qk_global(q_raw, kv_raw, w_q, w_k, [0, 0])
    np.testing.assert_allclose(q, ref_norm(q_raw, w_q), rtol=0, atol=1e-13)
    np.testing.assert_allclose(k, ref_norm(kv_raw, w_k), rtol=0, atol=1e-13)
    q_raw, k_raw, v_raw = raw(12, (2, 16, 256)), raw(13, (2, 8, 256)), raw(14, (2, 8, 256))
    w_q, w_k = weights(15, 256)
    q, k, v = oracle.decode_step_qkv_sliding(q_raw, k_raw, v_raw, w_q, w_k, [0, 0])
    np.testing.assert_allclose(k, ref_norm(k_raw, w_k), rtol=0, atol=1e-13)
    np.testing.assert_allclose(v, ref_norm(v_raw), rtol=0, atol=1e-13)


def test_global_inactive_pairs_are_not_rotated():
    # only pairs (i, i + 256) with i < 64 turn on global layers: coordinates
    # 64..255 and 320..511 keep the weighted norm's value at any position
    kv_raw = raw(16, (len(POSITIONS), 1, 512))
    w_q, w_k = weights(17, 512)
    _, k = oracle.decode_step_qk_global(raw(18, (len(POSITIONS), 16, 512)), kv_raw, w_q, w_k, POSITIONS)
    n = ref_norm(kv_raw, w_k)
    keep = np.r_[64:256, 320:512]
    np.testing.assert_allclose(k[..., keep], n[..., keep], rtol=0, atol=1e-13)
    # ... and pair 63 does turn at position 1: by 10^6^(-126/512) radians
    ang = 1e6 ** (-126.0 / 512)
    want = n[1, 0, 63] * np.cos(ang) - n[1, 0, 319] * np.sin(ang)
    assert abs(k[1, 0, 63] - want) < 1e-13


def test_prenorm_decode_matches_independent_pipeline():
    assert err_prenorm() < 1e-12


def test_prenorm_single_key_and_position_zero():
    # one cached token: the output is v = unit-norm x whatever k is; two
    # tokens: the first sits at position 0 (k unrotated), checked through
    # the softmax weights against the closed form
    q, cache, w_k, bt, lens, xs = prenorm_case(seq_lens=(1, 2), start=(0, 0), seed=19)
    got = oracle.paged_decode_global_prenorm(q, cache, w_k, bt, lens, "f32")
    np.testing.assert_allclose(got[0], np.broadcast_to(ref_norm(xs[0][0, 0]), (16, 512)), atol=1e-14)
    x = xs[1][:, 0]
    k0 = ref_norm(x[0], w_k)
    k1 = ref_rope(ref_norm(x[1], w_k), np.array(1), "global")
    qq = q[1].astype(np.float64)
    s0, s1 = qq @ k0, qq @ k1
    p1 = 1.0 / (1.0 + np.exp(s0 - s1))
    want = (1 - p1)[:, None] * ref_norm(x[0])[None] + p1[:, None] * ref_norm(x[1])[None]
    np.testing.assert_allclose(got[1], want, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

def _patch_const(mp, kind, **change):
    if kind == "global":
        mp.setattr(A, "GLOBAL_ROPE", {**A.GLOBAL_ROPE, **change})
        mp.setattr(P, "PRENORM_ROPE", {**P.PRENORM_ROPE, **change})
    else:
        mp.setattr(A, "SLIDING_ROPE", {**A.SLIDING_ROPE, **change})


def _rope_before_norm(mp, module):
    # the norm is skipped where it stands and applied after the rotation,
    # with the weight of the call it belongs to
    pending = []
    mp.setattr(module, "rmsnorm", lambda eps, x, w: (pending.append(w), x)[1])
    mp.setattr(module, "rope", lambda pos, x, **kw: NR.rmsnorm(EPS, NR.rope(pos=pos, x=x, **kw), pending.pop(0)))


def _wq_for_k(mp):
    # a decode step normalises q, then k: the k call gets the q call's weight
    calls = []

    def rms(eps, x, w):
        calls.append(w)
        return NR.rmsnorm(eps, x, calls[len(calls) - 1 - (len(calls) + 1) % 2])
    mp.setattr(A, "rmsnorm", rms)


MUTANTS = {
    "global theta 1e4": (lambda mp: _patch_const(mp, "global", theta=1e4), (err_step_global, err_prenorm)),
    "global active 128": (lambda mp: _patch_const(mp, "global", active=128), (err_step_global, err_prenorm)),
    "global active 256 (full RoPE)": (lambda mp: _patch_const(mp, "global", active=256), (err_step_global, err_prenorm)),
    "global denom 256": (lambda mp: _patch_const(mp, "global", denom=256), (err_step_global, err_prenorm)),
    "sliding theta 1e6": (lambda mp: _patch_const(mp, "sliding", theta=1e6), (err_step_sliding,)),
    "sliding active 64": (lambda mp: _patch_const(mp, "sliding", active=64), (err_step_sliding,)),
    "w_q used for k": (_wq_for_k, (err_step_global, err_step_sliding)),
    "RoPE before the norm (decode step)": (lambda mp: _rope_before_norm(mp, A), (err_step_global, err_step_sliding)),
    "RoPE before the norm (pre-norm decode)": (lambda mp: _rope_before_norm(mp, P), (err_prenorm,)),
    "k without its weight (pre-norm decode)": (
        lambda mp: mp.setattr(P, "rmsnorm", lambda eps, x, w: NR.rmsnorm_unit(eps, x)), (err_prenorm,)),
    "v through the weighted norm (pre-norm decode)": (
        lambda mp: mp.setattr(P, "rmsnorm_unit", lambda eps, x: NR.rmsnorm(eps, x, prenorm_case()[2])),
        (err_prenorm,)),
    "v without its norm (pre-norm decode)": (
        lambda mp: mp.setattr(P, "rmsnorm_unit", lambda eps, x: np.asarray(x, np.float64)), (err_prenorm,)),
    "v without its norm (sliding step)": (
        lambda mp: mp.setattr(A, "rmsnorm_unit", lambda eps, x: np.asarray(x, np.float64)), (err_step_sliding,)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    plant, pins = MUTANTS[name]
    with monkeypatch.context() as mp:
        plant(mp)
        worst = max(pin() for pin in pins)
    assert worst > 1e-4, f"{name}: pins still pass (max error {worst:.2e})"
    # and the unplanted oracle passes them again
    assert max(pin() for pin in pins) < 1e-11
