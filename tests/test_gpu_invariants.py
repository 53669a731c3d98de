"""Invariants of the decode kernels that hold at any size, checked on the GPU
through the C ABI (Op Specs of google/gemma-4-12B, Attention.lean: the
softmax weights are non-negative and sum to 1 over the visible positions, so
every output coordinate is a convex combination of the visible value rows):

* convexity: for every (b, h, d), min over visible l of v[l, d] <= o <= max;
* affine in V (sliding, separate v cache): v -> a*v + c gives o -> a*o + c;
  with a = 2, c = 0 the kernel's fp32 arithmetic scales exactly, so the
  output doubles bit for bit.
"""

import numpy as np
import pytest

import oracle
from workloads import inputs as I

from gpu_util import F32_TOL, global_on_gpu, sliding_on_gpu

pytestmark = pytest.mark.gpu


def visible_bounds_sliding(wl):
    lo = np.full(wl.q.shape, np.inf)
    hi = np.full(wl.q.shape, -np.inf)
    for b, L in enumerate(wl.seq_lens):
        a, e = oracle.sliding_visible_range(L, wl.window)
        if e <= a:
            continue
        v = oracle.stored_to_f64(oracle.gather_rowmajor_cache(wl.v_cache, wl.block_table[b], np.arange(a, e)),
                                 wl.kv_dtype)  # [n, Hkv, D]
        vr = np.repeat(v, wl.G, axis=1)        # query head c*G+g reads KV head c
        lo[b], hi[b] = vr.min(axis=0), vr.max(axis=0)
    return lo, hi


def visible_bounds_global(wl):
    lo = np.full(wl.q.shape, np.inf)
    hi = np.full(wl.q.shape, -np.inf)
    for b, L in enumerate(wl.seq_lens):
        if L <= 0:
            continue
        v = oracle.stored_to_f64(oracle.gather_tiled_cache(wl.kv_cache, wl.block_table[b], np.arange(L)),
                                 wl.kv_dtype)[:, 0]
        lo[b], hi[b] = v.min(axis=0), v.max(axis=0)
    return lo, hi


def assert_convex(got, lo, hi, slack, label):
    span = np.where(np.isfinite(hi - lo), hi - lo, 0.0)
    below = np.max(np.where(np.isfinite(lo), lo - got, -np.inf))
    above = np.max(np.where(np.isfinite(hi), got - hi, -np.inf))
    print(f"[invariants] {label}: worst excursion below {below:.2e}, above {above:.2e} "
          f"(slack {slack:.1e}, mean span {span.mean():.2f})", flush=True)
    assert below <= slack and above <= slack, label


@pytest.mark.parametrize("mode", ["config", "q_zero", "q_small"])
def test_sliding_output_is_convex_in_visible_values(gpu_lib, mode):
    kw = {"config": {}, "q_zero": dict(q_zero=True), "q_small": dict(q_scale=1 / 16)}[mode]
    wl = I.make_sliding([1, 17, 1000, 1025, 1039, 5000], kv_dtype="bf16", tag=(1200,), **I.SLIDING, **kw)
    got = sliding_on_gpu(wl)
    lo, hi = visible_bounds_sliding(wl)
    assert_convex(got, lo, hi, 1e-5, f"sliding {mode}")


@pytest.mark.parametrize("num_splits", [0, 1, 7])
@pytest.mark.parametrize("mode", ["config", "q_zero"])
def test_global_output_is_convex_in_visible_values(gpu_lib, mode, num_splits):
    kw = {"config": {}, "q_zero": dict(q_zero=True)}[mode]
    wl = I.make_global([1, 16, 300, 5000, 20000], kv_dtype="bf16", tag=(1201,), **I.GLOBAL, **kw)
    got = global_on_gpu(wl, num_splits)
    lo, hi = visible_bounds_global(wl)
    # p enters the PV product as bf16 hi + lo (about 2^-17 relative), while
    # the denominator sums the fp32 weights
    assert_convex(got, lo, hi, 1e-4, f"global {mode}, splits {num_splits}")


def test_sliding_doubling_v_doubles_output_bitwise(gpu_lib):
    wl = I.make_sliding([1, 17, 1000, 1025, 3000], kv_dtype="bf16", tag=(1202,), **I.SLIDING)
    o1 = sliding_on_gpu(wl)
    v2 = wl.v_cache.copy()
    finite = (v2 & 0x7F80) != 0x7F80          # leave NaN / Inf guard values alone
    f = oracle.stored_to_f64(v2[finite], "bf16") * 2.0
    v2[finite] = (f.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # exact: a power of 2
    wl2 = type(wl)(wl.q, wl.k_cache, v2, wl.block_table, wl.seq_lens, wl.window, wl.kv_dtype,
                   wl.Hkv, wl.G, wl.D)
    o2 = sliding_on_gpu(wl2)
    np.testing.assert_array_equal(o2, 2.0 * o1)


def test_sliding_fp32_affine_in_v(gpu_lib):
    wl = I.config_workload(0)  # fp32 KV
    o1 = sliding_on_gpu(wl)
    a, c = np.float32(-1.5), np.float32(0.25)
    v2 = wl.v_cache.copy()
    ok = np.isfinite(v2)
    v2[ok] = a * v2[ok] + c
    wl2 = type(wl)(wl.q, wl.k_cache, v2, wl.block_table, wl.seq_lens, wl.window, wl.kv_dtype,
                   wl.Hkv, wl.G, wl.D)
    o2 = sliding_on_gpu(wl2)
    err = float(np.max(np.abs(o2 - (float(a) * o1 + float(c)))))
    print(f"[invariants] fp32 affine in v: max deviation {err:.2e}", flush=True)
    assert err <= 2 * F32_TOL
