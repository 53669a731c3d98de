"""fp64 definitions of the per-head normalisations, the rotary embedding and
the sigmoid output gate around decode attention (test infrastructure only).

Each function restates one definition over NumPy float64:

* Op Specs page of google/gemma-4-12B, ``Norm.lean``: ``rms``, ``rmsnorm``
  (weight applied as ``w``) and ``rmsnormUnit`` (no weight);
* the same page, ``Rope.lean``: ``invFreq`` and ``rope`` (rotate-half RoPE on
  the pairs ``(i, i + rot/2)``, ``i < rot/2``; coordinates from ``rot`` on are
  left alone; frequencies with ``i >= active`` are 0);
* the same page, ``Attention.lean``: ``sigmoidGate``; and the Op Specs
  overview page, "Scalar functions": ``sigmoid``.

Rows are the last axis; any leading axes index (token, head) pairs, as the
pages allow for per-head norms.
"""

import numpy as np


def rms(eps, x):
    """``rms eps x``: sqrt(sum_j x_j^2 / H + eps) over the last axis (kept)."""
    x = np.asarray(x, dtype=np.float64)
    H = x.shape[-1]
    return np.sqrt(np.sum(x * x, axis=-1, keepdims=True) / H + eps)


def rmsnorm(eps, x, w):
    """``rmsnorm eps x w``: x / rms(x) * w (w over the last axis)."""
    return np.asarray(x, dtype=np.float64) / rms(eps, x) * np.asarray(w, dtype=np.float64)


def rmsnorm_unit(eps, x):
    """``rmsnormUnit eps x``: x / rms(x), no weight."""
    return np.asarray(x, dtype=np.float64) / rms(eps, x)


def inv_freq(theta, denom, active, i):
    """``invFreq theta denom active i``: theta^(-2i/denom) for i < active, else 0."""
    i = np.asarray(i)
    return np.where(i < active, np.power(float(theta), -(2.0 * i.astype(np.float64)) / denom), 0.0)


def rope(theta, rot, denom, active, pos, x):
    """``rope theta rot denom active pos x`` on rows x[..., D] at positions
    ``pos`` (broadcast against x.shape[:-1]).

    With half = rot/2 and a_i = pos * invFreq(i):
      out[i]        = x[i] cos a_i - x[i + half] sin a_i      (i < half)
      out[i + half] = x[i + half] cos a_i + x[i] sin a_i      (i < half)
      out[d]        = x[d]                                    (d >= 2*half)
    (the Lean term's ``else 0`` for a partner past D cannot occur when
    rot <= D).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = rot // 2
    assert 2 * half <= D
    pos = np.asarray(pos, dtype=np.float64)[..., None]
    i = np.arange(half)
    a = pos * inv_freq(theta, denom, active, i)
    c, s = np.cos(a), np.sin(a)
    out = x.copy()
    lo, hi = x[..., :half], x[..., half:2 * half]
    out[..., :half] = lo * c - hi * s
    out[..., half:2 * half] = hi * c + lo * s
    return out


def sigmoid(x):
    """``sigmoid x``: 1 / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def sigmoid_gate(o, gate):
    """``sigmoidGate o gate``: o * sigmoid(gate), elementwise."""
    return np.asarray(o, dtype=np.float64) * sigmoid(gate)
