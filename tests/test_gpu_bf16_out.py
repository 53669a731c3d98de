"""bf16 output of the decode calls (da_shape.out_dtype = bf16), on the GPU
through the C ABI.

Each output element is computed in fp32 exactly as for fp32 output and
rounded to nearest even once, so the bf16 output must equal the fp32
output rounded that way, bit for bit, on every path: sliding, global
(whole sequences written by the decode kernel, split ones by the merge),
gated (the gate applied before the one rounding), pre-norm and the
allocation-free global call. The rounded output is also checked against
the oracle, within the bf16 tolerance plus half an ulp.
"""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
import oracle
from workloads import inputs as I

from gpu_util import BF16_TOL, dev

pytestmark = pytest.mark.gpu


def rne(t):
    return t.to(torch.bfloat16)


def assert_rounded(o32, o16, label):
    ref = rne(o32)
    same = torch.equal(ref.view(torch.int16), o16.view(torch.int16))
    if not same:
        diff = (ref.view(torch.int16) != o16.view(torch.int16)).sum().item()
        print(f"[bf16 out] {label}: {diff} elements differ from the rounded fp32 output", flush=True)
    assert same, label


def half_ulp(o):
    """Half a bf16 ulp of every element (the rounding's own error bound)."""
    a = np.abs(o).astype(np.float64)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def check_oracle(o16, ref, label):
    got = o16.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref) - half_ulp(ref)
    worst = float(err.max()) if err.size else 0.0
    print(f"[bf16 out] {label}: max |err| beyond half an ulp {worst:.2e}", flush=True)
    assert worst <= BF16_TOL, label


def sliding_args(wl):
    return [dev(x) for x in (wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens)]


def global_args(wl):
    return [dev(x) for x in (wl.q, wl.kv_cache, wl.block_table, wl.seq_lens)]


def test_sliding_bf16_out(gpu_lib):
    wl = I.make_sliding([0, 1, 17, 1000, 1025, 5000], kv_dtype="bf16", tag=(1300,), **I.SLIDING)
    q, k, v, bt, sl = sliding_args(wl)
    o32 = da.attn_decode_sliding(q, k, v, bt, sl, wl.window)
    o16 = da.attn_decode_sliding(q, k, v, bt, sl, wl.window, out=torch.empty_like(o32, dtype=torch.bfloat16))
    gate = dev(I.make_gate(wl.q.shape, tag=(1301,)))
    g32 = da.attn_decode_sliding_gated(q, k, v, bt, sl, wl.window, gate)
    g16 = da.attn_decode_sliding_gated(q, k, v, bt, sl, wl.window, gate,
                                       out=torch.empty_like(o32, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert_rounded(o32, o16, "sliding")
    assert_rounded(g32, g16, "sliding gated")
    ref = oracle.paged_decode_sliding(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.window,
                                      wl.kv_dtype)
    check_oracle(o16, ref, "sliding")


@pytest.mark.parametrize("num_splits", [0, 1, 7])
def test_global_bf16_out(gpu_lib, num_splits):
    wl = I.make_global([0, 1, 16, 300, 5000, 20000], kv_dtype="bf16", tag=(1302,), **I.GLOBAL)
    q, kv, bt, sl = global_args(wl)
    o32 = da.attn_decode_global(q, kv, bt, sl, num_splits=num_splits)
    o16 = da.attn_decode_global(q, kv, bt, sl, num_splits=num_splits,
                                out=torch.empty_like(o32, dtype=torch.bfloat16))
    gate = dev(I.make_gate(wl.q.shape, tag=(1303,)))
    g32 = da.attn_decode_global_gated(q, kv, bt, sl, gate, num_splits=num_splits)
    g16 = da.attn_decode_global_gated(q, kv, bt, sl, gate, num_splits=num_splits,
                                      out=torch.empty_like(o32, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert_rounded(o32, o16, f"global, splits {num_splits}")
    assert_rounded(g32, g16, f"global gated, splits {num_splits}")
    ref = oracle.paged_decode_global(wl.q, wl.kv_cache, wl.block_table, wl.seq_lens, wl.kv_dtype)
    check_oracle(o16, ref, f"global, splits {num_splits}")
    check_oracle(g16, oracle.sigmoid_gate(ref, I.make_gate(wl.q.shape, tag=(1303,))),
                 f"global gated, splits {num_splits}")


def test_global_prenorm_and_noalloc_bf16_out(gpu_lib):
    pw = I.make_global_prenorm([1, 40, 700, 3000], tag=(1304,))
    args = [dev(x) for x in (pw.q, pw.x_cache, pw.w_k, pw.block_table, pw.seq_lens)]
    o32 = da.attn_decode_global_prenorm(*args)
    o16 = da.attn_decode_global_prenorm(*args, out=torch.empty_like(o32, dtype=torch.bfloat16))
    wl = I.make_global([3, 900, 12000], kv_dtype="bf16", tag=(1305,), **I.GLOBAL)
    q, kv, bt, sl = global_args(wl)
    n32 = da.attn_decode_global(q, kv, bt, sl)
    n16 = da.attn_decode_global_noalloc(q, kv, bt, sl, torch.empty_like(n32, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert_rounded(o32, o16, "pre-norm")
    assert_rounded(n32, n16, "no-alloc")
