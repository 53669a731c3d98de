"""Seeded random configurations of every call family against the fp64
oracle, on the GPU through the C ABI: batch sizes, lengths (0, page edges,
past the window), windows, KV-head counts, cache dtypes, splits and wave
counts drawn per case, each case small enough for the oracle to finish in
well under a second. The case's parameters are printed before it runs.

Bars: max-abs 2e-2 (bf16 KV) and 1e-5 (fp32 KV), as for the fixed tests.
"""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
import oracle
from workloads import inputs as I

from gpu_util import dev, max_abs, tol

pytestmark = pytest.mark.gpu

EDGES = [0, 1, 15, 16, 17, 31, 32, 33]


def draw_lens(rng, B, hi):
    """Lengths mixing page edges, small and large values."""
    out = []
    for _ in range(B):
        kind = rng.integers(3)
        if kind == 0:
            out.append(int(rng.choice(EDGES)))
        elif kind == 1:
            out.append(int(rng.integers(0, 200)))
        else:
            out.append(int(rng.integers(0, hi)))
    return out


@pytest.mark.parametrize("case", range(8))
def test_fuzz_sliding_decode(gpu_lib, case):
    rng = np.random.default_rng([1700, case])
    B = int(rng.integers(1, 13))
    Hkv = int(rng.choice([1, 2, 8]))
    kv_dtype = str(rng.choice(["bf16", "f32"]))
    window = int(rng.choice([0, 1, 16, 17, 100, 1024, 2048]))
    waves = int(rng.choice([0, 1, 2, 4] + ([8] if kv_dtype == "bf16" else [])))
    lens = draw_lens(rng, B, 3000)
    print(f"[fuzz sliding] case {case}: B={B} Hkv={Hkv} {kv_dtype} window={window} waves={waves} lens={lens}",
          flush=True)
    wl = I.make_sliding(lens, Hkv=Hkv, G=2, D=256, window=window, kv_dtype=kv_dtype, tag=(1700, case))
    args = [dev(x) for x in (wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens)]
    got = da.attn_decode_sliding(*args, window, num_splits=waves)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_sliding(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, window,
                                      kv_dtype)
    err = max_abs(got.cpu().numpy().astype(np.float64), ref)
    print(f"[fuzz sliding] case {case}: max-abs error {err:.3e}", flush=True)
    assert err <= tol(kv_dtype)


@pytest.mark.parametrize("case", range(8))
def test_fuzz_global_decode(gpu_lib, case):
    rng = np.random.default_rng([1701, case])
    B = int(rng.integers(1, 13))
    kv_dtype = str(rng.choice(["bf16", "f32"]))
    splits = int(rng.choice([0, 1, 2, 5, 33, 300]))
    lens = draw_lens(rng, B, 20000)
    print(f"[fuzz global] case {case}: B={B} {kv_dtype} splits={splits} lens={lens}", flush=True)
    wl = I.make_global(lens, kv_dtype=kv_dtype, tag=(1701, case), **I.GLOBAL)
    args = [dev(x) for x in (wl.q, wl.kv_cache, wl.block_table, wl.seq_lens)]
    got = da.attn_decode_global(*args, num_splits=splits)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_global(wl.q, wl.kv_cache, wl.block_table, wl.seq_lens, kv_dtype)
    err = max_abs(got.cpu().numpy().astype(np.float64), ref)
    print(f"[fuzz global] case {case}: max-abs error {err:.3e}", flush=True)
    assert err <= tol(kv_dtype)


@pytest.mark.parametrize("case", range(8))
def test_fuzz_multiquery(gpu_lib, case):
    rng = np.random.default_rng([1702, case])
    kind = "sliding" if case % 2 == 0 else "global"
    B = int(rng.integers(1, 7))
    splits = int(rng.choice([0, 0, 1, 3]))
    if kind == "sliding":
        Hkv = (1, 3, 8, 2)[(case // 2) % 4]
        window = (1, 17, 300, 1024)[(case // 2) % 4]  # window 1: exact (each query sees its own key)
        # counts below and above 128 queries (the two sliding kernels)
        counts = [int(rng.choice([0, 1, 8, 63, 64, 65, 127, 128, 129, 200, 300])) for _ in range(B)]
        shape = dict(Hkv=Hkv, G=2, D=256, window=window)
    else:
        counts = [int(rng.choice([0, 1, 7, 8, 9, 16, 40])) for _ in range(B)]
        shape = dict(I.GLOBAL)
    lens = [max(int(x), c if rng.integers(4) else 0) for x, c in zip(draw_lens(rng, B, 3000), counts)]
    print(f"[fuzz multiquery] case {case}: {kind} {shape} splits={splits} lens={lens} counts={counts}", flush=True)
    mq = I.make_multiquery(kind, lens, counts, tag=(1702, case), **shape)
    base = mq.base
    args = [dev(mq.q), dev(mq.q_start), max(mq.max_queries, 1)]
    tail = [dev(base.block_table), dev(base.seq_lens)]
    if kind == "sliding":
        got = da.attn_multiquery_sliding(*args, dev(base.k_cache), dev(base.v_cache), *tail, base.window,
                                         num_splits=splits)
        ref = oracle.paged_multiquery_sliding(mq.q, mq.q_start, base.k_cache, base.v_cache, base.block_table,
                                              base.seq_lens, base.window, base.kv_dtype)
    else:
        got = da.attn_multiquery_global(*args, dev(base.kv_cache), *tail, num_splits=splits)
        ref = oracle.paged_multiquery_global(mq.q, mq.q_start, base.kv_cache, base.block_table, base.seq_lens,
                                             base.kv_dtype)
    torch.cuda.synchronize()
    err = max_abs(got.cpu().numpy().astype(np.float64), ref)
    print(f"[fuzz multiquery] case {case}: max-abs error {err:.3e}", flush=True)
    assert np.isfinite(got.cpu().numpy()).all()
    assert err <= tol(base.kv_dtype)


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_every_sequence_empty(gpu_lib, kv_dtype):
    # no cached token anywhere: every output row is 0, for both decode calls,
    # at the default split and at explicit ones (the global merge then sees
    # only empty pieces); pre-filled outputs make sure the rows are written
    lens = [0, 0, 0]
    sl = I.make_sliding(lens, kv_dtype=kv_dtype, tag=(1703,), **I.SLIDING)
    gl = I.make_global(lens, kv_dtype=kv_dtype, tag=(1704,), **I.GLOBAL)
    s_args = [dev(x) for x in (sl.q, sl.k_cache, sl.v_cache, sl.block_table, sl.seq_lens)]
    g_args = [dev(x) for x in (gl.q, gl.kv_cache, gl.block_table, gl.seq_lens)]
    for splits in (0, 1, 5):
        so = torch.full((3, 16, 256), 7.0, device="cuda")
        go = torch.full((3, 16, 512), 7.0, device="cuda")
        da.attn_decode_sliding(*s_args, sl.window, out=so)
        da.attn_decode_global(*g_args, out=go, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.count_nonzero(so) == 0 and torch.count_nonzero(go) == 0, splits
