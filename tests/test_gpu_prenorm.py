"""GPU parity of attn_decode_global_prenorm (global decode that derives
k = rope(rmsnorm(x, w_k)) and v = rmsnormUnit(x) from the cached pre-norm
projection x) against the fp64 oracle, through the C ABI.

Bar: max-abs 2e-2 (bf16 cache, fp32 accumulate and output).
"""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
import oracle
from workloads import inputs as I

from gpu_util import BF16_TOL, dev, max_abs, oracle_rows_parallel

pytestmark = pytest.mark.gpu


def run(wl, num_splits=0):
    o = da.attn_decode_global_prenorm(dev(wl.q), dev(wl.x_cache), dev(wl.w_k), dev(wl.block_table),
                                      dev(wl.seq_lens), num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64)


def ref(wl, rows=None):
    rows = np.arange(len(wl.seq_lens)) if rows is None else np.asarray(rows)
    return oracle.paged_decode_global_prenorm(wl.q[rows], wl.x_cache, wl.w_k, wl.block_table[rows],
                                              wl.seq_lens[rows], wl.kv_dtype)


def check(wl, label, num_splits=0, rows=None):
    print(f"[prenorm] {label}: B={len(wl.seq_lens)} splits={num_splits}", flush=True)
    got = run(wl, num_splits)
    rows = np.arange(len(wl.seq_lens)) if rows is None else np.asarray(rows)
    err = max_abs(got[rows], ref(wl, rows))
    print(f"[prenorm] {label}: max-abs error {err:.3e}", flush=True)
    assert np.isfinite(got).all(), label
    assert err <= BF16_TOL, (label, err)
    return got


@pytest.mark.parametrize("num_splits", [0, 1, 3, 64, 1000])
def test_ragged_lengths(gpu_lib, num_splits):
    wl = I.make_global_prenorm([0, 1, 2, 15, 16, 17, 100, 1000, 4097, 333], tag=(960,))
    got = check(wl, "ragged", num_splits)
    assert np.all(got[0] == 0)


def test_many_short_sequences(gpu_lib):
    lens = np.random.default_rng(961).integers(1, 48, size=200)
    wl = I.make_global_prenorm(lens, tag=(961,))
    check(wl, "short sequences", 17)


def test_single_token_is_its_unit_norm_row(gpu_lib):
    wl = I.make_global_prenorm([1, 1], tag=(962,))
    got = run(wl)
    for b in range(2):
        x = oracle.stored_to_f64(oracle.gather_prenorm_cache(wl.x_cache, wl.block_table[b], [0])[0, 0], "bf16")
        want = x / np.sqrt(np.mean(x * x) + 1e-6)
        assert max_abs(got[b], np.broadcast_to(want, (16, 512))) <= 1e-5


def test_split_invariance_and_determinism(gpu_lib):
    wl = I.make_global_prenorm([5000, 1, 20000, 7777], tag=(963,))
    outs = [run(wl, s) for s in (1, 2, 5, 37, 256, 0)]
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= 2e-4
    assert np.array_equal(run(wl, 37), outs[3])
    assert max_abs(outs[0], ref(wl)) <= BF16_TOL


def test_far_positions(gpu_lib):
    # RoPE angles at positions up to ~150000 (the model's domain reaches 2^18)
    wl = I.make_global_prenorm([150001, 70000], tag=(964,))
    check(wl, "far positions")


def test_full_size_every_row(gpu_lib):
    sl = I.uniform_seq_lens((2,), 64, 1, 32768)
    wl = I.make_global_prenorm(sl, tag=(965,), P_max=2048)
    print("[prenorm] B=64 U[1,32768]: splits=0", flush=True)
    got = run(wl, 0)
    want = oracle_rows_parallel(lambda b: ref(wl, [b])[0], range(64))
    err = max_abs(got, want)
    print(f"[prenorm] B=64 U[1,32768]: max-abs error {err:.3e} over 64 of 64 sequences", flush=True)
    assert np.isfinite(got).all()
    assert err <= BF16_TOL


def test_append_into_prenorm_cache_then_decode(gpu_lib):
    """attn_kv_append_global_prenorm: q as the oracle's decode-step q (within
    one bf16 ulp), the new token's projection stored as bf16(x) in its slot of
    the pre-norm layout with every other byte of the cache unchanged, and the
    pre-norm decode over the appended cache against the oracle."""
    L = np.array([0, 15, 16, 17, 300, 4095], dtype=np.int32)  # new token at position L
    wl = I.make_global_prenorm(L + 1, tag=(960,))               # pages with room for it
    B, Hq, D = len(L), 16, 512
    rng = np.random.default_rng(961)
    q_raw = (rng.standard_normal((B, Hq, D)) * 2.0).astype(np.float32)
    x_raw = (rng.standard_normal((B, 1, D)) * 3.0).astype(np.float32)
    w_q = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    print(f"[prenorm append] B={B} positions={list(L)}", flush=True)
    xc = dev(wl.x_cache)
    q_out = da.attn_kv_append_global_prenorm(dev(q_raw), dev(x_raw), dev(w_q), dev(wl.block_table), dev(L), xc)
    torch.cuda.synchronize()
    q_bits = q_out.cpu().view(torch.int16).numpy().view(np.uint16)
    cache = xc.cpu().view(torch.int16).numpy().view(np.uint16)

    q_ref, _ = oracle.decode_step_qk_global(q_raw.astype(np.float64), x_raw.astype(np.float64),
                                            w_q.astype(np.float64), w_q.astype(np.float64), L)
    got_q = oracle.stored_to_f64(q_bits, "bf16")
    ulp = np.abs(got_q) * 2.0 ** -7 + 1e-30
    assert (np.abs(got_q - q_ref) <= np.maximum(ulp, np.abs(q_ref) * 2.0 ** -7)).all()

    expected = wl.x_cache.copy()
    for b in range(B):
        I.scatter_prenorm(expected, wl.block_table[b], [int(L[b])], I.to_storage(x_raw[b:b + 1].astype(np.float64), "bf16"))
    np.testing.assert_array_equal(cache, expected)

    o = da.attn_decode_global_prenorm(q_out, xc, dev(wl.w_k), dev(wl.block_table), dev(L + 1))
    torch.cuda.synchronize()
    ref_o = oracle.paged_decode_global_prenorm(q_bits, expected, wl.w_k, wl.block_table, L + 1, "bf16")
    err = max_abs(o.cpu().numpy().astype(np.float64), ref_o)
    print(f"[prenorm append] decode after append: max-abs error {err:.3e}", flush=True)
    assert err <= BF16_TOL
