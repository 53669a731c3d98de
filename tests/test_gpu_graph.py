"""A decode step captured into a HIP graph (how a serving loop replays it):
every replay must reproduce the eager outputs, with eager work and
synchronisations between replays. The calls record kernel launches only (no
memset nodes). The global split depends only on the lengths and the number
of workgroups (one per compute unit by default, or the caller's count), and
the merge folds pieces in a fixed order, so every replay matches the eager
outputs bit for bit, also with the workspace of another stream."""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
from workloads import inputs as I

from gpu_util import dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu_lib):
    sl = I.make_sliding([1, 17, 1500, 4000, 333], kv_dtype="bf16", tag=(420,), **I.SLIDING)
    gl = I.make_global([1, 300, 9000, 20000, 17], kv_dtype="bf16", tag=(421,), **I.GLOBAL)
    d_sl = [dev(x) for x in (sl.q, sl.k_cache, sl.v_cache, sl.block_table, sl.seq_lens)]
    d_gl = [dev(x) for x in (gl.q, gl.kv_cache, gl.block_table, gl.seq_lens)]
    o_sl = torch.empty(tuple(d_sl[0].shape), dtype=torch.float32, device="cuda")
    o_gl = torch.empty(tuple(d_gl[0].shape), dtype=torch.float32, device="cuda")
    o_gd = torch.empty(tuple(d_gl[0].shape), dtype=torch.float32, device="cuda")

    def step():
        da.attn_decode_sliding(*d_sl, sl.window, out=o_sl)
        da.attn_decode_global(*d_gl, out=o_gl, num_splits=64)
        da.attn_decode_global(*d_gl, out=o_gd)

    step()
    torch.cuda.synchronize()
    ref_sl, ref_gl, ref_gd = o_sl.cpu().numpy(), o_gl.cpu().numpy(), o_gd.cpu().numpy()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    other = I.make_global([5000, 2], kv_dtype="bf16", tag=(422,), **I.GLOBAL)
    d_other = [dev(x) for x in (other.q, other.kv_cache, other.block_table, other.seq_lens)]
    for replay in range(4):
        for o in (o_sl, o_gl, o_gd):
            o.fill_(float("nan"))
        da.attn_decode_global(*d_other)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {replay}", flush=True)
        assert np.array_equal(o_sl.cpu().numpy(), ref_sl), replay
        assert np.array_equal(o_gl.cpu().numpy(), ref_gl), replay
        assert np.array_equal(o_gd.cpu().numpy(), ref_gd), replay
