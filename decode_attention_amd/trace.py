"""Per-workgroup timeline of the global decode call (measurement support, not
part of the attention path): ``attn_decode_global_traced`` from
include/decode_attn_trace.h runs the global call's kernels and has every
workgroup of the decode kernel record its start and end time, its XCC and
its page count.

``summarize`` and ``format_summary`` turn the entries into start and end
statistics (overall and per XCC); ``python -m workloads.trace_run`` prints
them for the benchmark's global workloads.
"""

import ctypes

import numpy as np

from .binding import (_check, _check_common, _global_shape, _ptr, _stream, attn_decode_global_workspace_bytes,
                      load_library)

TICK_US = 0.01  # the real-time counter runs at 100 MHz


def _lib():
    lib = load_library()
    if not getattr(lib, "_trace_ready", False):
        vp = ctypes.c_void_p
        from .binding import DaShape
        lib.attn_decode_global_traced.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(DaShape), vp, ctypes.c_size_t,
                                                  vp, vp]
        lib.attn_decode_global_traced.restype = ctypes.c_int32
        lib._trace_ready = True
    return lib


def global_timeline(q, kv_cache, block_table, seq_lens, out, num_splits=0, stream=None):
    """Runs the global call once with the timeline; returns (out, entries)
    with entries int64 [splits, 4] as the header describes them."""
    import torch
    lib = _lib()
    _check_common(q, block_table, seq_lens, (kv_cache,))
    shape = _global_shape(q, kv_cache, block_table, num_splits)
    need = attn_decode_global_workspace_bytes(shape)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    splits = num_splits if num_splits > 0 else torch.cuda.get_device_properties(q.device).multi_processor_count
    tr = torch.zeros((splits, 4), dtype=torch.int64, device=q.device)
    _check(lib.attn_decode_global_traced(_ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), _ptr(out),
                                         ctypes.byref(shape), _ptr(ws), need, _ptr(tr), _stream(stream)))
    torch.cuda.synchronize()
    return out, tr.cpu().numpy()


def summarize(entries):
    """Start and end times (µs from the first start), per-XCC means."""
    t0 = entries[:, 0].min()
    start = (entries[:, 0] - t0) * TICK_US
    end = (entries[:, 1] - t0) * TICK_US
    xcc = entries[:, 2] & 0xF
    segs = entries[:, 2] >> 8
    pages = entries[:, 3] & 0xFFFFFFFF
    res = {
        "workgroups": int(len(entries)),
        "start_max_us": float(start.max()),
        "end_mean_us": float(end.mean()),
        "end_p10_us": float(np.percentile(end, 10)),
        "end_p50_us": float(np.median(end)),
        "end_p90_us": float(np.percentile(end, 90)),
        "end_max_us": float(end.max()),
        "busy_fraction": float((end - start).sum() / (len(end) * end.max())),
        "pages_per_workgroup": (int(pages.min()), int(pages.max())),
        "segments_mean": float(segs.mean()),
        "per_xcc_end_mean_us": {int(x): float(end[xcc == x].mean()) for x in sorted(set(xcc.tolist()))},
        "per_xcc_end_max_us": {int(x): float(end[xcc == x].max()) for x in sorted(set(xcc.tolist()))},
    }
    # end time by segments flushed, relative to the mean end of the same XCC
    # (a workgroup's extra segments against the XCCs' different speeds)
    rel = end.copy()
    for x in set(xcc.tolist()):
        rel[xcc == x] -= end[xcc == x].mean()
    res["end_vs_xcc_mean_by_segments_us"] = {int(k): (int((segs == k).sum()), float(rel[segs == k].mean()))
                                             for k in sorted(set(segs.tolist()))}
    return res


def format_summary(label, res, event_us=None, pages_total=None):
    lines = [f"{label}: {res['workgroups']} workgroups, {res['pages_per_workgroup'][0]}-"
             f"{res['pages_per_workgroup'][1]} pages each, {res['segments_mean']:.2f} segments on average"]
    if event_us is not None:
        lines.append(f"  call by HIP events (back to back): {event_us:.1f} us")
    lines.append(f"  last start {res['start_max_us']:.1f} us; end mean {res['end_mean_us']:.1f}, p10 "
                 f"{res['end_p10_us']:.1f}, p50 {res['end_p50_us']:.1f}, p90 {res['end_p90_us']:.1f}, "
                 f"max {res['end_max_us']:.1f} us; busy {100 * res['busy_fraction']:.1f}% of workgroups x span")
    if pages_total:
        lines.append(f"  decode kernel span {res['end_max_us']:.1f} us = "
                     f"{pages_total * 16384 / res['end_max_us'] / 1e3:.0f} GB/s of KV; at the mean end "
                     f"{pages_total * 16384 / res['end_mean_us'] / 1e3:.0f} GB/s")
    lines.append("  per XCC mean end: " + " ".join(f"{x}:{v:.1f}" for x, v in res["per_xcc_end_mean_us"].items()))
    lines.append("  per XCC max end:  " + " ".join(f"{x}:{v:.1f}" for x, v in res["per_xcc_end_max_us"].items()))
    lines.append("  end vs its XCC's mean, by segments: " + " ".join(
        f"{k}: {v[1]:+.1f} us (n={v[0]})" for k, v in res["end_vs_xcc_mean_by_segments_us"].items()))
    return "\n".join(lines)
