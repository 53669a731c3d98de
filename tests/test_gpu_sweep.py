"""GPU parity on the full decode-step sweep's shapes: B = 256 sequences with
lengths log-uniform in [1, 131072], a sliding layer (Hkv 8, G 2, D 256,
window 1024) and a global layer (Hkv 1, G 16, D 512, K = V), caches drawn on
the device (workloads.inputs.device_layer). The oracle computes
sampled sequences from their stored bytes, copied back from the device.

Bar: max-abs 2e-2 for bf16 KV (fp32 accumulate, fp32 out).
"""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
import oracle
from workloads import inputs as I

from gpu_util import BF16_TOL, max_abs

pytestmark = pytest.mark.gpu


def sampled_rows(seq_lens):
    order = np.argsort(seq_lens, kind="stable")
    picks = [order[0], order[1], order[len(order) // 2], order[-2], order[-1], 0, 77, 255]
    return np.unique(np.asarray(picks, dtype=np.int64))


@pytest.mark.parametrize("layer", [0, 5, 11, 46])
def test_sweep_layer_full_size_sampled(gpu_lib, layer):
    kind = I.sweep_kind(layer)
    sl = I.sweep_seq_lens()
    print(f"[sweep] layer {layer} ({kind}): B={len(sl)}, L in [{sl.min()}, {sl.max()}]", flush=True)
    dl = I.device_layer(kind, sl, layer=layer)
    if kind == "sliding":
        out = da.attn_decode_sliding(dl.q, *dl.caches, dl.block_table, dl.seq_lens, dl.window)
    else:
        out = da.attn_decode_global(dl.q, *dl.caches, dl.block_table, dl.seq_lens)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    rows = sampled_rows(sl)
    h = I.sample_to_host(dl, rows)
    if kind == "sliding":
        ref = oracle.paged_decode_sliding(h.q, h.k_cache, h.v_cache, h.block_table, h.seq_lens, h.window, "bf16")
    else:
        ref = oracle.paged_decode_global(h.q, h.kv_cache, h.block_table, h.seq_lens, "bf16")
    err = max_abs(got[rows], ref)
    print(f"[sweep] layer {layer}: max-abs error {err:.3e} over rows {rows.tolist()}", flush=True)
    assert err <= BF16_TOL
    del dl, out
    torch.cuda.empty_cache()
