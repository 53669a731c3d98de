"""Bound calls (decode_attention_amd.bind): the library calls of a checked
call, replayed on the same tensors. On the GPU through the C ABI: a bound
call's results equal the plain call's bit for bit, and a replay reads the
buffers' current contents (new query rows give the new outputs)."""

import numpy as np
import torch

import decode_attention_amd as da
from workloads import inputs as I

from gpu_util import dev

import pytest

pytestmark = pytest.mark.gpu


def test_bound_decode_calls_match_and_reread_their_inputs(gpu_lib):
    sl = I.make_sliding([1, 100, 2000, 5000], kv_dtype="bf16", tag=(1500,), **I.SLIDING)
    gl = I.make_global([1, 300, 5000, 20000], kv_dtype="bf16", tag=(1501,), **I.GLOBAL)
    s_args = [dev(x) for x in (sl.q, sl.k_cache, sl.v_cache, sl.block_table, sl.seq_lens)]
    g_args = [dev(x) for x in (gl.q, gl.kv_cache, gl.block_table, gl.seq_lens)]
    s_ref = da.attn_decode_sliding(*s_args, sl.window)
    g_ref = da.attn_decode_global(*g_args)
    s_out = torch.empty_like(s_ref)
    g_out = torch.empty_like(g_ref)
    run_s, o1 = da.bind(da.attn_decode_sliding, *s_args, sl.window, out=s_out)
    run_g, o2 = da.bind(da.attn_decode_global, *g_args, out=g_out)
    torch.cuda.synchronize()
    assert o1 is s_out and o2 is g_out
    assert torch.equal(s_out, s_ref) and torch.equal(g_out, g_ref)
    s_out.zero_()
    g_out.zero_()
    run_s()
    run_g()
    torch.cuda.synchronize()
    assert torch.equal(s_out, s_ref) and torch.equal(g_out, g_ref)
    # new query rows in the same buffers: the replay sees them
    s_args[0].copy_(torch.flip(s_args[0], dims=[0]))
    g_args[0].copy_(torch.flip(g_args[0], dims=[0]))
    run_s()
    run_g()
    s_new = da.attn_decode_sliding(*s_args, sl.window)
    g_new = da.attn_decode_global(*g_args)
    torch.cuda.synchronize()
    assert torch.equal(s_out, s_new) and torch.equal(g_out, g_new)
    assert not torch.equal(g_new, g_ref)


def test_bound_appends_match(gpu_lib):
    aw = I.make_append("global", [5, 900, 4000], kv_dtype="bf16", tag=(1502,), **I.GLOBAL)
    d = [dev(x) for x in (aw.q_raw, aw.k_raw, aw.w_q, aw.w_k, aw.block_table, aw.positions, aw.k_cache)]
    d2 = [t.clone() for t in d]
    q_ref = da.attn_kv_append_global(*d)
    q_out = torch.empty_like(q_ref)
    run, res = da.bind(da.attn_kv_append_global, *d2, q_out=q_out)
    run()
    torch.cuda.synchronize()
    assert res is q_out
    assert torch.equal(q_out.view(torch.int16), q_ref.view(torch.int16))
    assert torch.equal(d2[-1].view(torch.int16), d[-1].view(torch.int16))  # the same cache bytes
