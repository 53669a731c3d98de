"""attn_decode_global_noalloc (the global decode on the library's own device
scratch array) against attn_decode_global (caller-provided workspace), through
the C ABI: two calls in a row on the same scratch, the second with a smaller
batch, each bit for bit equal to the workspace call with the same split; the
explicit-split limit is refused on the host."""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
from workloads import inputs as I

from gpu_util import BF16_TOL, dev, max_abs

pytestmark = pytest.mark.gpu


def run_both(wl, num_splits):
    q, kv, bt, sl = (dev(x) for x in (wl.q, wl.kv_cache, wl.block_table, wl.seq_lens))
    ref = da.attn_decode_global(q, kv, bt, sl, num_splits=num_splits)
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device="cuda")
    da.attn_decode_global_noalloc(q, kv, bt, sl, out, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.parametrize("num_splits", [0, 7, 256])
def test_noalloc_matches_workspace_call_twice(gpu_lib, num_splits):
    import oracle
    big = I.make_global([0, 5000, 1, 20000, 333, 16, 7777, 2], kv_dtype="bf16", tag=(1300,), **I.GLOBAL)
    small = I.make_global([40, 1200], kv_dtype="bf16", tag=(1301,), **I.GLOBAL)
    for label, wl in (("first, B=8", big), ("second, B=2", small)):
        print(f"[noalloc] {label}: splits={num_splits}", flush=True)
        got, ref = run_both(wl, num_splits)
        assert np.isfinite(got).all(), label
        np.testing.assert_array_equal(got, ref)
        want = oracle.paged_decode_global(wl.q, wl.kv_cache, wl.block_table, wl.seq_lens, "bf16")
        assert max_abs(got.astype(np.float64), want) <= BF16_TOL, label


def test_noalloc_refuses_splits_beyond_its_scratch(gpu_lib):
    wl = I.make_global([100, 200], kv_dtype="bf16", tag=(1302,), **I.GLOBAL)
    q, kv, bt, sl = (dev(x) for x in (wl.q, wl.kv_cache, wl.block_table, wl.seq_lens))
    out = torch.zeros(tuple(q.shape), dtype=torch.float32, device="cuda")
    with pytest.raises(da.DecodeAttnError) as e:
        da.attn_decode_global_noalloc(q, kv, bt, sl, out, num_splits=257)
    assert e.value.status == -3  # DA_ERR_WORKSPACE, nothing enqueued
