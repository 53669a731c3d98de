"""GPU parity of the gated decode calls (attention output times
sigmoid(gate), fused into the kernels' final writes) against the fp64
oracle's decode followed by its sigmoidGate, through the C ABI.

Bars: those of the ungated calls (max-abs 2e-2 for bf16 KV, 1e-5 for fp32
KV), since |sigmoid| <= 1 and the gate adds about one fp32 rounding. Two
gate values give exact results in fp32: 0 (sigmoid 1/2, out = o / 2) and
+-1e4 (sigmoid 1 and 0).
"""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
import oracle
from workloads import inputs as I

from gpu_util import BF16_TOL, dev, global_on_gpu, max_abs, oracle_rows_parallel, sliding_on_gpu, tol

pytestmark = pytest.mark.gpu


def sliding_gated_on_gpu(wl, gate):
    q, k, v = dev(wl.q), dev(wl.k_cache), dev(wl.v_cache)
    bt, sl = dev(wl.block_table), dev(wl.seq_lens)
    o = da.attn_decode_sliding_gated(q, k, v, bt, sl, wl.window, dev(gate))
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64)


def global_gated_on_gpu(wl, gate, num_splits=0):
    q, kv = dev(wl.q), dev(wl.kv_cache)
    bt, sl = dev(wl.block_table), dev(wl.seq_lens)
    o = da.attn_decode_global_gated(q, kv, bt, sl, dev(gate), num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64)


def sliding_ref(wl, gate):
    o = oracle.paged_decode_sliding(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                                    wl.window, wl.kv_dtype)
    return oracle.sigmoid_gate(o, gate)


def global_ref(wl, gate, rows):
    o = oracle.paged_decode_global(wl.q[rows], wl.kv_cache, wl.block_table[rows], wl.seq_lens[rows],
                                   wl.kv_dtype)
    return oracle.sigmoid_gate(o, gate[rows])


@pytest.mark.parametrize("cfg", [0, 1])
def test_sliding_gated_configs(gpu_lib, cfg):
    wl = I.config_workload(cfg)
    gate = I.make_gate(wl.q.shape, tag=(600, cfg))
    print(f"[gate] sliding config {cfg}", flush=True)
    err = max_abs(sliding_gated_on_gpu(wl, gate), sliding_ref(wl, gate))
    print(f"[gate] sliding config {cfg}: max-abs error {err:.3e}", flush=True)
    assert err <= tol(wl.kv_dtype)


def test_sliding_gated_edges(gpu_lib):
    wl = I.make_sliding([0, 1, 16, 17, 1025, 3000], kv_dtype="bf16", tag=(601,), **I.SLIDING)
    gate = I.make_gate(wl.q.shape, tag=(601,))
    print("[gate] sliding edges", flush=True)
    got = sliding_gated_on_gpu(wl, gate)
    assert max_abs(got, sliding_ref(wl, gate)) <= BF16_TOL
    assert np.all(got[0] == 0)


def test_sliding_gate_exact_values(gpu_lib):
    wl = I.make_sliding([5, 900, 2500], kv_dtype="bf16", tag=(602,), **I.SLIDING)
    print("[gate] sliding exact gate values", flush=True)
    plain = sliding_on_gpu(wl)
    np.testing.assert_array_equal(sliding_gated_on_gpu(wl, np.zeros(wl.q.shape, np.float32)), plain / 2)
    np.testing.assert_array_equal(sliding_gated_on_gpu(wl, np.full(wl.q.shape, 1e4, np.float32)), plain)
    assert np.all(sliding_gated_on_gpu(wl, np.full(wl.q.shape, -1e4, np.float32)) == 0)


# splits 1: every sequence is finished inside one workgroup (the kernel's own
# write); many splits: most rows are written by the merge.
@pytest.mark.parametrize("num_splits", [0, 1, 7, 300])
def test_global_gated_ragged(gpu_lib, num_splits):
    wl = I.make_global([0, 1, 2, 15, 16, 17, 100, 1000, 4097, 333], kv_dtype="bf16", tag=(603,), **I.GLOBAL)
    gate = I.make_gate(wl.q.shape, tag=(603,))
    print(f"[gate] global ragged, splits {num_splits}", flush=True)
    rows = np.arange(len(wl.seq_lens))
    got = global_gated_on_gpu(wl, gate, num_splits)
    err = max_abs(got, global_ref(wl, gate, rows))
    print(f"[gate] global ragged, splits {num_splits}: max-abs error {err:.3e}", flush=True)
    assert err <= BF16_TOL
    assert np.all(got[0] == 0)


@pytest.mark.parametrize("num_splits", [1, 0])
def test_global_gate_exact_values(gpu_lib, num_splits):
    wl = I.make_global([3, 700, 9000], kv_dtype="bf16", tag=(604,), **I.GLOBAL)
    print(f"[gate] global exact gate values, splits {num_splits}", flush=True)
    plain = global_on_gpu(wl, num_splits)
    zero = np.zeros(wl.q.shape, np.float32)
    np.testing.assert_array_equal(global_gated_on_gpu(wl, zero, num_splits), plain / 2)
    np.testing.assert_array_equal(global_gated_on_gpu(wl, zero + 1e4, num_splits), plain)
    assert np.all(global_gated_on_gpu(wl, zero - 1e4, num_splits) == 0)


def test_global_gated_full_size_every_row(gpu_lib):
    wl = I.config_workload(2)
    gate = I.make_gate(wl.q.shape, tag=(605,))
    print("[gate] global full size", flush=True)
    got = global_gated_on_gpu(wl, gate)
    ref = oracle_rows_parallel(lambda b: global_ref(wl, gate, [b])[0], range(64))
    err = max_abs(got, ref)
    print(f"[gate] global full size: max-abs error {err:.3e}", flush=True)
    assert err <= BF16_TOL
