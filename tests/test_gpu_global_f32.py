"""GPU parity of attn_decode_global on an fp32 K=V cache (the fp32 kernel:
every product in fp32 on mfma_f32_16x16x4f32) against the fp64 oracle,
through the C ABI.

Bar: max-abs 1e-5 for fp32 KV. The oracle reads the same stored fp32
values; the kernel's error is fp32 rounding of the dot products, the
exponentials and the running sums.
"""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
import oracle
from workloads import inputs as I

from gpu_util import F32_TOL, dev, global_on_gpu, max_abs, oracle_rows_parallel

pytestmark = pytest.mark.gpu


def check(wl, label, num_splits=0):
    print(f"[global f32] {label}: B={len(wl.seq_lens)} splits={num_splits}", flush=True)
    got = global_on_gpu(wl, num_splits)
    ref = oracle_rows_parallel(lambda b: oracle.paged_decode_global(
        wl.q[b:b + 1], wl.kv_cache, wl.block_table[b:b + 1], wl.seq_lens[b:b + 1], wl.kv_dtype)[0],
        range(len(wl.seq_lens)))
    err = max_abs(got, ref)
    print(f"[global f32] {label}: max-abs error {err:.3e}", flush=True)
    assert np.isfinite(got).all(), label
    assert err <= F32_TOL, (label, err)
    return got, ref


SMALL = [0, 1, 2, 15, 16, 17, 31, 33, 100, 1000, 4097, 333]


@pytest.mark.parametrize("num_splits", [0, 1, 2, 3, 7, 64, 1000])
def test_ragged_lengths_every_split(gpu_lib, num_splits):
    wl = I.make_global(SMALL, kv_dtype="f32", tag=(1400,), **I.GLOBAL)
    got, _ = check(wl, "ragged", num_splits)
    assert np.all(got[0] == 0)  # no cached token: all-zero rows


@pytest.mark.parametrize("num_splits", [0, 3, 100])
def test_many_short_sequences(gpu_lib, num_splits):
    # 1-3 pages per sequence: two-page steps straddle sequence starts, and
    # workgroup ranges cut sequences at odd page offsets
    rng = np.random.default_rng(1401)
    wl = I.make_global(rng.integers(1, 48, size=200), kv_dtype="f32", tag=(1401,), **I.GLOBAL)
    check(wl, f"short sequences, splits {num_splits}", num_splits)


def test_lengths_of_the_b64_workload(gpu_lib):
    # 16 sequences drawn like the B = 64 benchmark's lengths (uniform in
    # [1, 32768]), every row against the oracle
    wl = I.make_global(I.uniform_seq_lens((1402,), 16, 1, 32768), kv_dtype="f32", tag=(1402,), **I.GLOBAL)
    check(wl, "lengths U[1, 32768]")


def test_split_invariance(gpu_lib):
    # all products fp32: splits differ by fp32 summation order only
    wl = I.make_global([5000, 1, 20000, 7777], kv_dtype="f32", tag=(1403,), **I.GLOBAL)
    outs = [global_on_gpu(wl, s) for s in (1, 2, 5, 37, 256, 0)]
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= 2e-6


@pytest.mark.parametrize("mode", ["q_zero", "q_small"])
def test_diffuse_softmax(gpu_lib, mode):
    # q = 0: every visible key weighs the same, the output is the mean of the
    # visible value rows; a small q keeps the weights nearly flat
    kw = dict(q_zero=True) if mode == "q_zero" else dict(q_scale=1.0 / np.sqrt(512))
    wl = I.make_global([1, 17, 700, 9000], kv_dtype="f32", tag=(1404,), **kw, **I.GLOBAL)
    got, _ = check(wl, mode, 0)
    if mode == "q_zero":
        for b, L in enumerate(wl.seq_lens):
            v = oracle.stored_to_f64(oracle.gather_tiled_cache(wl.kv_cache, wl.block_table[b], np.arange(L)),
                                     wl.kv_dtype)[:, 0]
            assert max_abs(got[b], np.broadcast_to(v.mean(axis=0), got[b].shape)) <= F32_TOL


def test_gated_bf16_out_and_noalloc(gpu_lib):
    wl = I.make_global([3, 900, 12000, 40], kv_dtype="f32", tag=(1405,), **I.GLOBAL)
    q, kv, bt, sl = (dev(x) for x in (wl.q, wl.kv_cache, wl.block_table, wl.seq_lens))
    gate_np = I.make_gate(wl.q.shape, tag=(1406,))
    gate = dev(gate_np)
    o32 = da.attn_decode_global(q, kv, bt, sl)
    o16 = da.attn_decode_global(q, kv, bt, sl, out=torch.empty_like(o32, dtype=torch.bfloat16))
    g32 = da.attn_decode_global_gated(q, kv, bt, sl, gate)
    na = da.attn_decode_global_noalloc(q, kv, bt, sl, torch.empty_like(o32))
    torch.cuda.synchronize()
    ref = oracle.paged_decode_global(wl.q, wl.kv_cache, wl.block_table, wl.seq_lens, wl.kv_dtype)
    assert max_abs(o32.cpu().numpy().astype(np.float64), ref) <= F32_TOL
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
    gref = oracle.sigmoid_gate(ref, gate_np)
    assert max_abs(g32.cpu().numpy().astype(np.float64), gref) <= F32_TOL
    assert torch.equal(na, o32)
