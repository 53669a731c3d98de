"""The traced global call (include/decode_attn_trace.h): same output as
attn_decode_global bit for bit, and a timeline entry per workgroup that
covers the batch's pages."""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
from workloads import inputs as I
from decode_attention_amd import trace as T

from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("num_splits", [0, 5, 300])
def test_traced_call_matches_and_covers_the_pages(gpu_lib, num_splits):
    wl = I.make_global([1, 17, 5000, 300, 0, 4097], kv_dtype="bf16", tag=(1400,), **I.GLOBAL)
    args = [dev(x) for x in (wl.q, wl.kv_cache, wl.block_table, wl.seq_lens)]
    print(f"[trace] splits={num_splits}", flush=True)
    ref = da.attn_decode_global(*args, num_splits=num_splits)
    out = torch.empty_like(ref)
    out, e = T.global_timeline(*args, out, num_splits=num_splits)
    assert torch.equal(out, ref)
    splits = num_splits or torch.cuda.get_device_properties(0).multi_processor_count
    assert e.shape == (splits, 4)
    assert np.all(e[:, 1] >= e[:, 0]) and np.all(e[:, 0] > 0)
    pages = int(((wl.seq_lens.astype(np.int64) + 15) // 16).sum())
    assert int((e[:, 3] & 0xFFFFFFFF).sum()) == pages
    assert np.all((e[:, 2] & 0xF) < 8)
    res = T.summarize(e)
    assert res["end_max_us"] >= res["end_mean_us"] >= 0
