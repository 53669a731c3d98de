"""GPU parity of the decode-step norm + RoPE + cache append
(attn_kv_append_sliding / attn_kv_append_global) against the fp64 oracle,
through the C ABI.

Bar: stored bf16 values within one bf16 ulp of the oracle's real value (the
kernel computes in fp32 and rounds once; the oracle's value can sit on the
other side of a rounding midpoint only by much less than that), fp32 values
within 1e-5; every other cache element bit-for-bit unchanged.
"""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
import oracle
from workloads import inputs as I

from gpu_util import BF16_TOL, dev, max_abs

pytestmark = pytest.mark.gpu


def ulp_bf16(ref):
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_close(got_stored, ref, kv_dtype, label):
    got = oracle.stored_to_f64(got_stored, kv_dtype)
    if kv_dtype == "bf16":
        bad = np.abs(got - ref) > ulp_bf16(ref)
        assert not bad.any(), (label, int(bad.sum()), float(np.max(np.abs(got - ref))))
    else:
        assert max_abs(got, ref) <= 1e-5, (label, max_abs(got, ref))


def host(t):
    a = t.cpu()
    return a.view(torch.int16).numpy().view(np.uint16) if a.dtype == torch.bfloat16 else a.numpy()


def run_append(wl):
    q_raw, k_raw = dev(wl.q_raw), dev(wl.k_raw)
    w_q, w_k = dev(wl.w_q), dev(wl.w_k)
    bt, pos = dev(wl.block_table), dev(wl.positions)
    kc = dev(wl.k_cache)
    if wl.kind == "sliding":
        vc = dev(wl.v_cache)
        q_out = da.attn_kv_append_sliding(q_raw, k_raw, dev(wl.v_raw), w_q, w_k, bt, pos, kc, vc)
        torch.cuda.synchronize()
        return host(q_out), host(kc), host(vc)
    q_out = da.attn_kv_append_global(q_raw, k_raw, w_q, w_k, bt, pos, kc)
    torch.cuda.synchronize()
    return host(q_out), host(kc), None


def check_append(wl, label):
    print(f"[append] {label}: {wl.kind} {wl.kv_dtype} B={len(wl.positions)} positions={list(wl.positions)}", flush=True)
    q_out, kc, vc = run_append(wl)
    valid = (wl.positions >= 0) & (wl.positions < wl.block_table.shape[1] * 16)
    if wl.kind == "sliding":
        q, k, v = oracle.decode_step_qkv_sliding(wl.q_raw, wl.k_raw, wl.v_raw, wl.w_q, wl.w_k, wl.positions)
    else:
        q, k = oracle.decode_step_qk_global(wl.q_raw, wl.k_raw, wl.w_q, wl.w_k, wl.positions)
    assert_close(q_out[valid], q[valid], wl.kv_dtype, label + " q")
    pages, slots = oracle.append_targets(wl.block_table[valid], wl.positions[valid])
    k_keep, v_keep = wl.k_cache.copy(), (wl.v_cache.copy() if vc is not None else None)
    kc_cmp, vc_cmp = kc.copy(), (vc.copy() if vc is not None else None)
    for i, b in enumerate(np.nonzero(valid)[0]):
        if wl.kind == "sliding":
            assert_close(kc[pages[i], :, slots[i], :], k[b], wl.kv_dtype, label + f" k[{b}]")
            assert_close(vc[pages[i], :, slots[i], :], v[b], wl.kv_dtype, label + f" v[{b}]")
            for a in (k_keep, kc_cmp, v_keep, vc_cmp):
                a[pages[i], :, slots[i], :] = 0
        else:
            got = kc[pages[i], :, :, slots[i], :].reshape(wl.Hkv, wl.D)
            assert_close(got, k[b], wl.kv_dtype, label + f" k[{b}]")
            for a in (k_keep, kc_cmp):
                a[pages[i], :, :, slots[i], :] = 0
    # nothing else was written
    np.testing.assert_array_equal(kc_cmp.view(np.uint8), k_keep.view(np.uint8))
    if vc is not None:
        np.testing.assert_array_equal(vc_cmp.view(np.uint8), v_keep.view(np.uint8))
    return q_out


POS_SLIDING = [0, 1, 15, 16, 17, 1023, 4095, 4096, 262143]
POS_GLOBAL = [0, 15, 16, 31, 1000, 32767, 131071, 262143]


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_sliding_append(gpu_lib, kv_dtype):
    wl = I.make_append("sliding", POS_SLIDING, Hkv=8, G=2, D=256, kv_dtype=kv_dtype, tag=(501,))
    check_append(wl, "sliding")


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_global_append(gpu_lib, kv_dtype):
    wl = I.make_append("global", POS_GLOBAL, Hkv=1, G=16, D=512, kv_dtype=kv_dtype, tag=(502,))
    check_append(wl, "global")


def test_other_head_counts(gpu_lib):
    wl = I.make_append("sliding", [3, 40, 500], Hkv=2, G=4, D=256, tag=(503,))
    check_append(wl, "Hkv=2 G=4")
    wl = I.make_append("global", [3, 40, 500], Hkv=2, G=8, D=512, tag=(504,))
    check_append(wl, "global Hkv=2 G=8")


def test_positions_out_of_range_leave_everything_untouched(gpu_lib):
    wl = I.make_append("sliding", [-1, 5, 64, 7], Hkv=8, G=2, D=256, tag=(505,), P_max=4)
    # positions -1 and 64 (= 16 * P_max) are outside the block-table rows
    q_out = check_append(wl, "out of range")
    assert q_out.shape[0] == 4


def test_append_then_decode_sliding(gpu_lib):
    base = I.make_sliding([5, 100, 1023, 1031, 2003], tag=(506,), Hkv=8, G=2, D=256, window=1024)
    wl = I.make_append("sliding", base.seq_lens, Hkv=8, G=2, D=256, tag=(507,), block_table=base.block_table,
                       k_cache=base.k_cache, v_cache=base.v_cache)
    q_out, kc, vc = run_append(wl)
    seq_lens = base.seq_lens + 1
    got = da.attn_decode_sliding(dev(q_out), dev(kc), dev(vc), dev(base.block_table), dev(seq_lens),
                                 base.window).cpu().numpy().astype(np.float64)
    # the oracle's own path: its fp64 q, k, v rounded once to bf16 and stored
    q, k, v = oracle.decode_step_qkv_sliding(wl.q_raw, wl.k_raw, wl.v_raw, wl.w_q, wl.w_k, wl.positions)
    k_exp, v_exp = base.k_cache.copy(), base.v_cache.copy()
    pages, slots = oracle.append_targets(base.block_table, wl.positions)
    for b in range(len(seq_lens)):
        k_exp[pages[b], :, slots[b], :] = oracle.f64_to_bf16_bits(k[b])
        v_exp[pages[b], :, slots[b], :] = oracle.f64_to_bf16_bits(v[b])
    ref = oracle.paged_decode_sliding(oracle.f64_to_bf16_bits(q), k_exp, v_exp, base.block_table, seq_lens,
                                      base.window, "bf16")
    assert max_abs(got, ref) <= BF16_TOL


def test_append_then_decode_global(gpu_lib):
    base = I.make_global([7, 300, 5001], tag=(508,), Hkv=1, G=16, D=512)
    wl = I.make_append("global", base.seq_lens, Hkv=1, G=16, D=512, tag=(509,), block_table=base.block_table,
                       k_cache=base.kv_cache)
    q_out, kc, _ = run_append(wl)
    seq_lens = base.seq_lens + 1
    got = da.attn_decode_global(dev(q_out), dev(kc), dev(base.block_table), dev(seq_lens)).cpu().numpy()
    q, k = oracle.decode_step_qk_global(wl.q_raw, wl.k_raw, wl.w_q, wl.w_k, wl.positions)
    kv_exp = base.kv_cache.copy()
    pages, slots = oracle.append_targets(base.block_table, wl.positions)
    for b in range(len(seq_lens)):
        kv_exp[pages[b], :, :, slots[b], :] = oracle.f64_to_bf16_bits(k[b]).reshape(1, 64, 8)
    ref = oracle.paged_decode_global(oracle.f64_to_bf16_bits(q), kv_exp, base.block_table, seq_lens, "bf16")
    assert max_abs(got.astype(np.float64), ref) <= BF16_TOL
