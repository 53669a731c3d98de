"""GPU parity of attn_decode_sliding against the fp64 oracle, through the C ABI.

Bars: max-abs 1e-5 for fp32 KV, 2e-2 for bf16 KV (fp32 accumulate, fp32 out).
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as I

from gpu_util import dev, max_abs, sliding_on_gpu, tol

pytestmark = pytest.mark.gpu


def check(wl, label):
    print(f"[sliding] {label}: B={len(wl.seq_lens)} dtype={wl.kv_dtype} window={wl.window}", flush=True)
    got = sliding_on_gpu(wl)
    ref = oracle.paged_decode_sliding(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                                      wl.window, wl.kv_dtype)
    err = max_abs(got, ref)
    print(f"[sliding] {label}: max-abs error {err:.3e}", flush=True)
    assert np.isfinite(got).all(), label
    assert err <= tol(wl.kv_dtype), (label, err)
    return got, ref


def test_config0_tiny_fp32(gpu_lib):
    check(I.config_workload(0), "config 0")


def test_config1_full_bf16(gpu_lib):
    check(I.config_workload(1), "config 1")


EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 33, 1000, 1023, 1024, 1025, 1039, 1040, 1041, 1056, 2047, 5000]


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_ragged_lengths_and_misaligned_windows(gpu_lib, kv_dtype):
    wl = I.make_sliding(EDGE_LENS, kv_dtype=kv_dtype, tag=(300,), **I.SLIDING)
    got, _ = check(wl, f"edge lengths {kv_dtype}")
    assert np.all(got[0] == 0)  # L = 0


@pytest.mark.parametrize("window", [0, 1, 2, 7, 16, 17, 100, 511, 4096])
def test_other_windows(gpu_lib, window):
    wl = I.make_sliding([0, 1, 5, 16, 17, 40, 300, 1500], Hkv=8, G=2, D=256, window=window,
                        kv_dtype="bf16", tag=(301, window))
    got, _ = check(wl, f"window {window}")
    if window == 0:
        assert np.all(got == 0)


def test_window_one_returns_last_value_row(gpu_lib):
    wl = I.make_sliding([3, 20, 1030], Hkv=8, G=2, D=256, window=1, kv_dtype="f32", tag=(302,))
    got = sliding_on_gpu(wl)
    for b, L in enumerate(wl.seq_lens):
        v = oracle.gather_rowmajor_cache(wl.v_cache, wl.block_table[b], [L - 1])[0]  # [Hkv, D]
        np.testing.assert_array_equal(got[b], np.repeat(v.astype(np.float64), 2, axis=0))


@pytest.mark.parametrize("Hkv", [1, 3])
def test_other_kv_head_counts(gpu_lib, Hkv):
    wl = I.make_sliding([7, 900, 1100], Hkv=Hkv, G=2, D=256, window=1024, kv_dtype="bf16", tag=(303, Hkv))
    check(wl, f"Hkv={Hkv}")


@pytest.mark.parametrize("mode", ["q_zero", "q_small"])
def test_diffuse_softmax(gpu_lib, mode):
    kw = dict(q_zero=True) if mode == "q_zero" else dict(q_scale=1 / 16)
    wl = I.make_sliding([1, 64, 1024, 3000], kv_dtype="bf16", tag=(304,), **I.SLIDING, **kw)
    check(wl, mode)


def test_full_allocation_with_poisoned_history(gpu_lib):
    # Every page of the sequence allocated; positions before the window are NaN.
    wl = I.make_sliding([1100, 2048, 3001], kv_dtype="bf16", tag=(305,), window_only=False, **I.SLIDING)
    check(wl, "full allocation")


def test_deterministic_and_permutation_invariant(gpu_lib):
    seq = [1, 700, 1024, 1041, 4000]
    a = I.make_sliding(seq, kv_dtype="bf16", tag=(306,), **I.SLIDING)
    o1 = sliding_on_gpu(a)
    o2 = sliding_on_gpu(a)
    assert np.array_equal(o1, o2)
    # Same logical content, different physical placement.
    rng = np.random.default_rng(7)
    perm = rng.permutation(a.meta["num_pages"] - 1)
    inv = np.argsort(perm)
    k2 = a.k_cache.copy()
    v2 = a.v_cache.copy()
    k2[perm] = a.k_cache[:-1]
    v2[perm] = a.v_cache[:-1]
    bt2 = a.block_table.copy()
    used = bt2 != a.meta["num_pages"] - 1
    bt2[used] = perm[bt2[used]]
    del inv
    b = I.SlidingWorkload(a.q, k2, v2, bt2, a.seq_lens, a.window, a.kv_dtype, a.Hkv, a.G, a.D, a.meta)
    assert np.array_equal(sliding_on_gpu(b), o1)


def test_head_isolation_and_read_only(gpu_lib):
    a = I.make_sliding([200, 1500], kv_dtype="bf16", tag=(307,), **I.SLIDING)
    q, k, v = dev(a.q), dev(a.k_cache), dev(a.v_cache)
    bt, sl = dev(a.block_table), dev(a.seq_lens)
    import decode_attention_amd as da
    ksum, vsum = k.view(torch.int16).sum().item(), v.view(torch.int16).sum().item()
    base = da.attn_decode_sliding(q, k, v, bt, sl, a.window).cpu()
    torch.cuda.synchronize()
    assert k.view(torch.int16).sum().item() == ksum and v.view(torch.int16).sum().item() == vsum
    k2 = k.clone()
    k2[:, 3] = (k2[:, 3].float() * -2.0).to(torch.bfloat16)
    pert = da.attn_decode_sliding(q, k2, v, bt, sl, a.window).cpu()
    heads_c3 = [6, 7]
    others = [h for h in range(16) if h not in heads_c3]
    assert torch.equal(pert[:, others], base[:, others])
    assert not torch.equal(pert[:, heads_c3], base[:, heads_c3])


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_invariant_to_waves_per_unit(gpu_lib, kv_dtype):
    # The window of each (sequence, KV head) is divided among 1, 2, 4 or (bf16)
    # 8 waves, page by page, whose states are merged in LDS: every wave count
    # matches the oracle, the counts agree to fp32 rounding of the merge, and
    # each repeats bit for bit (a race in the LDS merge would show in one of
    # the three)
    wl = I.make_sliding(EDGE_LENS, kv_dtype=kv_dtype, tag=(1600,), **I.SLIDING)
    ref = oracle.paged_decode_sliding(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.window,
                                      wl.kv_dtype)
    args = [dev(x) for x in (wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens)]
    import decode_attention_amd as da
    outs = {}
    counts = (1, 2, 4, 8) if kv_dtype == "bf16" else (1, 2, 4)  # 8 waves: bf16 caches only
    for nw in counts:
        a = da.attn_decode_sliding(*args, wl.window, num_splits=nw)
        b = da.attn_decode_sliding(*args, wl.window, num_splits=nw)
        torch.cuda.synchronize()
        assert torch.equal(a, b), nw
        outs[nw] = a.cpu().numpy().astype(np.float64)
        err = max_abs(outs[nw], ref)
        print(f"[sliding] {kv_dtype}, {nw} waves per unit: max-abs error {err:.3e}", flush=True)
        assert err <= tol(kv_dtype), (nw, err)
    default = da.attn_decode_sliding(*args, wl.window).cpu().numpy().astype(np.float64)
    assert np.array_equal(default, outs[4])
    for nw in counts:
        assert max_abs(outs[nw], outs[4]) <= 2e-6, nw
