"""Helpers for GPU tests: move a host workload to the device and run the
library through its C ABI binding."""

import numpy as np
import torch

import decode_attention_amd as da

BF16_TOL = 2e-2   # max-abs error bound for bf16 KV (fp32 accumulate / output)
F32_TOL = 1e-5    # max-abs error bound for fp32 KV


def dev(a, kv_dtype=None, device="cuda"):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def sliding_on_gpu(wl, out=None):
    q, k, v = dev(wl.q), dev(wl.k_cache), dev(wl.v_cache)
    bt, sl = dev(wl.block_table), dev(wl.seq_lens)
    o = da.attn_decode_sliding(q, k, v, bt, sl, wl.window, out=out)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64)


def global_on_gpu(wl, num_splits=0):
    q, kv = dev(wl.q), dev(wl.kv_cache)
    bt, sl = dev(wl.block_table), dev(wl.seq_lens)
    o = da.attn_decode_global(q, kv, bt, sl, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64)


def tol(kv_dtype):
    return BF16_TOL if kv_dtype == "bf16" else F32_TOL


def oracle_rows_parallel(fn, rows, workers=16):
    """fn(row) -> oracle output of one sequence, for every row, computed in a
    thread pool (NumPy releases the GIL in its kernels); stacked in order."""
    import concurrent.futures
    rows = list(rows)
    with concurrent.futures.ThreadPoolExecutor(min(workers, max(1, len(rows)))) as ex:
        return np.stack(list(ex.map(fn, rows)))


def max_abs(a, b):
    return float(np.max(np.abs(a - b))) if a.size else 0.0
