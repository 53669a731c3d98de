#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step = one pass of the hot path over one batch at Gemma-4-12B shapes,
B = 64, seq_lens uniform in [1, 32768] (bf16 KV, fp32 accumulate and output):
  * attn_decode_sliding: sliding layer, 16 q heads on 8 KV heads, D = 256,
    window 1024, separate k/v caches (row-major pages);
  * attn_decode_global: global layer, 16 q heads on 1 KV head, D = 512,
    values = keys (tiled pages), split over workgroups + log-sum-exp merge.
Inputs are generated on the host, copied to HBM once, and are resident
before the timed region. The metric is achieved HBM GB/s over the algorithmic
bytes (KV read once, K=V counted once, plus q, out and block-table entries)
and microseconds per layer call.

Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth

# HBM bytes one attn_decode_global call moves on this workload (main kernel +
# merge kernel), from two rocprofv3 --pmc passes over this script: FETCH_SIZE
# scaled by 2.0 and WRITE_SIZE by 1.0, the factors that make the same counters
# read 512 MiB each for a 512 MiB device-to-device copy. Valid only for the
# kernel sources they were taken on (hash below); reported as null otherwise.
GLOBAL_TRAFFIC = {
    "sources": ("decode_attention_amd/csrc/global.hip", "decode_attention_amd/csrc/common.hpp"),
    "sha256": "606211f87b445b3f31c23dea36388e4e609bd4670291df2adc77369b3fa290f6",
    "bytes_per_call": 1172391776,
    # SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs) of
    # global_decode_kernel, from a third --pmc pass over the same sources
    "mfma_busy": 0.1211,
}
METRIC = "decode-attn achieved HBM GB/s (% of peak) + µs/layer, Gemma-4 shapes B=64"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sliding_bytes(wl):
    import numpy as np
    esize = 2 if wl.kv_dtype == "bf16" else 4
    L = wl.seq_lens.astype(np.int64)
    vis = np.minimum(L, wl.window)
    kv = int(vis.sum()) * wl.Hkv * wl.D * 2 * esize
    B, Hq = len(L), wl.Hkv * wl.G
    lo = np.maximum(L - wl.window, 0)
    pages = np.where(vis > 0, (L - 1) // 16 - lo // 16 + 1, 0)
    return dict(kv=kv, q=B * Hq * wl.D * esize, out=B * Hq * wl.D * 4,
                table=int(pages.sum()) * 4 + B * 4)


def global_bytes(wl):
    import numpy as np
    esize = 2 if wl.kv_dtype == "bf16" else 4
    L = wl.seq_lens.astype(np.int64)
    B, Hq = len(L), wl.Hkv * wl.G
    return dict(kv=int(L.sum()) * wl.Hkv * wl.D * esize, q=B * Hq * wl.D * esize,
                out=B * Hq * wl.D * 4, table=int(((L + 15) // 16).sum()) * 4 + B * 4)


def append_bytes(aw):
    """Algorithmic bytes of one decode-step append: fp32 projections, norm
    weights, positions and one block-table entry per sequence in; q and the
    new k (and v) rows out in the cache dtype."""
    esize = 2 if aw.kv_dtype == "bf16" else 4
    B, Hq = len(aw.positions), aw.Hkv * aw.G
    kv_rows = (2 if aw.v_raw is not None else 1) * B * aw.Hkv
    return (B * Hq + kv_rows) * aw.D * (4 + esize) + 2 * aw.D * 4 + 2 * B * 4


def multiquery_work(mq):
    """Algorithmic bytes (keys some query sees, read once, K = V once on
    global layers; q, fp32 out and block-table entries) and FLOPs (4 * D per
    visible (query, head, key)) of one multi-query call."""
    import numpy as np
    base = mq.base
    esize = 2
    sliding = mq.kind == "sliding"
    kv_bytes, flops, table = 0, 0, 0
    for b in range(len(base.seq_lens)):
        L, S = int(base.seq_lens[b]), int(mq.q_start[b + 1] - mq.q_start[b])
        if S <= 0 or L <= 0:
            continue
        pos = L - S + np.arange(S, dtype=np.int64)
        pos = pos[pos >= 0]
        if len(pos) == 0:
            continue
        lo = max(0, int(pos.min()) - base.window + 1) if sliding else 0
        n_keys = L - lo
        kv_bytes += n_keys * base.Hkv * base.D * esize * (2 if sliding else 1)
        table += ((L - 1) // 16 - lo // 16 + 1) * 4
        vis = np.minimum(pos + 1, base.window) if sliding else pos + 1
        flops += int(vis.sum()) * base.Hkv * base.G * base.D * 4
    T, Hq, D = mq.q.shape
    return kv_bytes + T * Hq * D * (esize + 4) + table, flops


def time_calls(fn, n):
    """Mean µs per call of fn over n back-to-back calls (HIP events on the
    current stream, after one untimed call)."""
    import torch
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def time_cold(fn, n, flush):
    """Median µs of fn over n calls, each after a 1 GiB write to `flush` that
    evicts L2 and the 256 MB Infinity Cache (events around fn only)."""
    import numpy as np
    import torch
    fn()
    times = []
    for i in range(n):
        flush.fill_(i & 0x7F)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(times))


def time_context(da, I, sl, gl, d_sl, d_gl, out_sl, out_gl, sb, gb, num_splits, oracle_threads, cpu_out):
    """Context for the step's numbers, timed after it: the read bandwidth the
    kernels' access pattern reaches (HBM probe), the calls with cold caches,
    and the long-context global call (B = 2, lengths 131072 and 262144).
    With oracle_threads > 0 the oracle is also timed on the long-context
    layer (both sequences, stored bytes copied back) into cpu_out."""
    import types
    import torch
    from decode_attention_amd import probe as P
    res = {}
    # probe: random 16 KB pages of a 4 GiB buffer, the decode kernels' loads
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device="cuda")
    n_pages = buf.numel() // P.PAGE_BYTES
    gen = torch.Generator(device="cpu").manual_seed(1234)
    ids = torch.randperm(n_pages, generator=gen).to(torch.int32).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.read_pages(buf, ids, 256, sink)  # checks the ids once
    best = (0.0, 0)
    for wg in (256, 512, 1024, 2048):
        us = time_calls(lambda: P.read_pages(buf, ids, wg, sink, check_ids=False), 10)
        gbs = n_pages * P.PAGE_BYTES / (us * 1e-6) / 1e9
        res[f"hbm_probe_{wg}wg_GBps"] = round(gbs, 1)
        best = max(best, (gbs, wg))
    res["hbm_probe_GBps"] = round(best[0], 1)
    res["hbm_probe_workload"] = ("4 GiB read as 16 KB pages in random order, 16-byte non-temporal loads, "
                                 f"best of 256-2048 workgroups ({best[1]})")
    del ids
    flush = buf[: 1 << 30]
    # cold caches: every call after a 1 GiB write
    s_cold = time_cold(lambda: da.attn_decode_sliding(*d_sl[:5], sl.window, out=out_sl), 10, flush)
    g_cold = time_cold(lambda: da.attn_decode_global(*d_gl, out=out_gl, num_splits=num_splits), 10, flush)
    res["sliding_us_cold_median"] = round(s_cold, 2)
    res["global_us_cold_median"] = round(g_cold, 2)
    res["sliding_GBps_cold"] = round(sum(sb.values()) / (s_cold * 1e-6) / 1e9, 1)
    res["global_GBps_cold"] = round(sum(gb.values()) / (g_cold * 1e-6) / 1e9, 1)
    # long-context global layer: two sequences, 24,576 pages
    dl = I.device_layer("global", [131072, 262144], tag=(3,))
    out = torch.empty((2, 16, 512), dtype=torch.float32, device="cuda")
    call = lambda: da.attn_decode_global(dl.q, *dl.caches, dl.block_table, dl.seq_lens, out=out,
                                         num_splits=num_splits)
    wl = types.SimpleNamespace(seq_lens=dl.host_seq_lens, window=0, kv_dtype="bf16", Hkv=1, G=16, D=512)
    lb = sum(global_bytes(wl).values())
    l_hot = time_calls(call, 20)
    l_cold = time_cold(call, 10, flush)
    res["long_context_workload"] = "global layer, B=2, seq_lens {131072, 262144}, caches drawn on the device"
    res["long_context_us_per_call"] = round(l_hot, 2)
    res["long_context_GBps"] = round(lb / (l_hot * 1e-6) / 1e9, 1)
    res["long_context_us_cold_median"] = round(l_cold, 2)
    res["long_context_GBps_cold"] = round(lb / (l_cold * 1e-6) / 1e9, 1)
    if oracle_threads > 0:
        h = I.sample_to_host(dl, [0, 1])
        t = time_oracle_rows(oracle_global_fn(h), [0, 1], oracle_threads)
        cpu_out["long_context_global_bf16_B2"] = {"seconds": round(t, 3), "GBps": round(lb / t / 1e9, 4),
                                                  "sample": "both sequences (one thread each)"}
        log(f"oracle: long context {t:.1f} s")
        del h
    log("context: " + ", ".join(f"{k}={v}" for k, v in res.items() if not k.endswith("workload")))
    del dl, out, buf, flush
    torch.cuda.empty_cache()
    return res


def counters_current():
    """True if the kernel sources are those the recorded counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in GLOBAL_TRAFFIC["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest() == GLOBAL_TRAFFIC["sha256"]


def to_dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_workers():
    """Threads the oracle baseline runs on: the cores this process may use,
    at most 16 (a one-GPU machine's share of its host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def time_oracle_rows(fn, rows, workers):
    """Wall seconds of fn(row) over every row, in a pool of `workers` threads
    with the BLAS pools pinned to one thread each (NumPy releases the GIL in
    its kernels, so the sequences run in parallel)."""
    import concurrent.futures
    from threadpoolctl import threadpool_limits
    rows = list(rows)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(min(workers, len(rows))) as ex:
            list(ex.map(fn, rows))
        return time.perf_counter() - t0


def oracle_sliding_fn(wl):
    import oracle
    return lambda b: oracle.paged_decode_sliding(wl.q[b:b + 1], wl.k_cache, wl.v_cache, wl.block_table[b:b + 1],
                                                 wl.seq_lens[b:b + 1], wl.window, wl.kv_dtype)


def oracle_global_fn(wl):
    import oracle
    return lambda b: oracle.paged_decode_global(wl.q[b:b + 1], wl.kv_cache, wl.block_table[b:b + 1],
                                                wl.seq_lens[b:b + 1], wl.kv_dtype)


def cpu_baseline(sl, gl, workers):
    """The oracle as it stands (fp64 NumPy) on the step's own workload, both
    calls in full (64 + 64 sequences), and on the tiny fp32 sliding case."""
    from workloads import inputs as I
    t_sl = time_oracle_rows(oracle_sliding_fn(sl), range(len(sl.seq_lens)), workers)
    t_gl = time_oracle_rows(oracle_global_fn(gl), range(len(gl.seq_lens)), workers)
    b_sl, b_gl = sum(sliding_bytes(sl).values()), sum(global_bytes(gl).values())
    tiny = I.config_workload(0)
    t_tiny = time_oracle_rows(oracle_sliding_fn(tiny), range(len(tiny.seq_lens)), workers)
    b_tiny = sum(sliding_bytes(tiny).values())
    log(f"oracle: sliding B=64 {t_sl:.2f} s, global B=64 {t_gl:.2f} s, tiny fp32 {t_tiny:.3f} s "
        f"on {workers} threads")
    return {
        "value": round((b_sl + b_gl) / (t_sl + t_gl) / 1e9, 4),
        "unit": "GB/s",
        "cores": int(workers),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"the whole step workload: all 64 sliding and all 64 global sequences, one sequence per "
                   f"task on {workers} threads (one BLAS thread each), fp64 NumPy; algorithmic bytes of "
                   f"both calls / wall time ({t_sl + t_gl:.1f} s)"),
        "workloads": {
            "tiny_sliding_fp32_B4": {"seconds": round(t_tiny, 6), "GBps": round(b_tiny / t_tiny / 1e9, 4),
                                     "sample": "all 4 sequences"},
            "sliding_bf16_B64": {"seconds": round(t_sl, 6), "GBps": round(b_sl / t_sl / 1e9, 4),
                                 "sample": "all 64 sequences"},
            "global_bf16_B64": {"seconds": round(t_gl, 6), "GBps": round(b_gl / t_gl / 1e9, 4),
                                "sample": "all 64 sequences"},
        },
    }


def time_extras(da, I, sl, gl, d_sl, d_gl, out_sl, out_gl, sb, gb, n_extra, num_splits):
    """The decode-step appends and the gated variants, timed after the step
    (not part of it): one new token per sequence at position L, the gate on
    the same outputs."""
    import numpy as np
    import torch
    log("timing the decode-step appends and the gated calls")
    shp = dict(Hkv=sl.Hkv, G=sl.G, D=sl.D)
    aws = I.make_append("sliding", sl.seq_lens, kv_dtype="bf16", tag=(700,), **shp)
    awg = I.make_append("global", gl.seq_lens, kv_dtype="bf16", tag=(701,), **I.GLOBAL)
    d_as = [to_dev(x) for x in (aws.q_raw, aws.k_raw, aws.v_raw, aws.w_q, aws.w_k, aws.block_table,
                                aws.positions, aws.k_cache, aws.v_cache)]
    d_ag = [to_dev(x) for x in (awg.q_raw, awg.k_raw, awg.w_q, awg.w_k, awg.block_table, awg.positions,
                                awg.k_cache)]
    q_as = torch.empty((64, 16, 256), dtype=torch.bfloat16, device="cuda")
    q_ag = torch.empty((64, 16, 512), dtype=torch.bfloat16, device="cuda")
    gate_sl = to_dev(I.make_gate(sl.q.shape, tag=(702,)))
    gate_gl = to_dev(I.make_gate(gl.q.shape, tag=(703,)))
    # bound calls (arguments checked once, as a serving loop would issue
    # them), and the same calls through the checked Python path
    run_as, _ = da.bind(da.attn_kv_append_sliding, *d_as, q_out=q_as)
    run_ag, _ = da.bind(da.attn_kv_append_global, *d_ag, q_out=q_ag)
    app_sl_us = time_calls(run_as, n_extra)
    app_gl_us = time_calls(run_ag, n_extra)
    app_sl_checked_us = time_calls(lambda: da.attn_kv_append_sliding(*d_as, q_out=q_as), n_extra)
    app_gl_checked_us = time_calls(lambda: da.attn_kv_append_global(*d_ag, q_out=q_ag), n_extra)
    gsl_us = time_calls(lambda: da.attn_decode_sliding_gated(*d_sl[:5], sl.window, gate_sl, out=out_sl), n_extra)
    ggl_us = time_calls(lambda: da.attn_decode_global_gated(*d_gl, gate_gl, out=out_gl,
                                                            num_splits=num_splits), n_extra)
    # several queries per sequence: 8 draft tokens per sequence (speculative
    # verification) at the decode workloads' lengths, and one 2048-token
    # prefill chunk per sequence of B = 4
    mq_sl = I.make_multiquery("sliding", sl.seq_lens, np.full(64, 8), tag=(704,), P_max=2048, **shp,
                              window=sl.window)
    q8 = I.rms_rows(I.rng_for((705,), 0, I.STREAM_MQ), (64 * 8, gl.Hkv * gl.G, gl.D))
    mq_gl = I.MultiQueryWorkload("global", I.to_storage(q8, "bf16"), np.arange(0, 65 * 8, 8, dtype=np.int32), gl)
    pf_sl = I.make_multiquery("sliding", [4096] * 4, [2048] * 4, tag=(706,), **shp, window=sl.window)
    pf_gl = I.make_multiquery("global", [8192] * 4, [2048] * 4, tag=(707,), **I.GLOBAL)
    mq_res = {}
    for name, mq in (("verify_sliding", mq_sl), ("verify_global", mq_gl), ("prefill_sliding", pf_sl),
                     ("prefill_global", pf_gl)):
        base = mq.base
        args = [to_dev(mq.q), to_dev(mq.q_start), mq.max_queries]
        tail = [to_dev(base.block_table), to_dev(base.seq_lens)]
        o = torch.empty(mq.q.shape, dtype=torch.float32, device="cuda")
        if mq.kind == "sliding":
            caches = [to_dev(base.k_cache), to_dev(base.v_cache)] if base is not sl else d_sl[1:3]
            fn = lambda: da.attn_multiquery_sliding(*args, *caches, *tail, base.window, out=o)
        else:
            caches = [d_gl[1]] if base is gl else [to_dev(base.kv_cache)]
            fn = lambda: da.attn_multiquery_global(*args, *caches, *tail, out=o)
        us = time_calls(fn, n_extra)
        nbytes, flops = multiquery_work(mq)
        mq_res[f"mq_{name}_us_per_call"] = round(us, 2)
        mq_res[f"mq_{name}_GBps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        mq_res[f"mq_{name}_TFLOPs"] = round(flops / (us * 1e-6) / 1e12, 2)
        del caches, fn, o
    log("multi-query: " + ", ".join(f"{k}={v}" for k, v in mq_res.items()))
    # global decode from the pre-norm projection at the global workload's lengths
    pw = I.make_global_prenorm(gl.seq_lens, tag=(708,), P_max=2048)
    d_pw = [to_dev(x) for x in (pw.q, pw.x_cache, pw.w_k, pw.block_table, pw.seq_lens)]
    o_pw = torch.empty((64, 16, 512), dtype=torch.float32, device="cuda")
    pre_us = time_calls(lambda: da.attn_decode_global_prenorm(*d_pw, out=o_pw, num_splits=num_splits), n_extra)
    mq_res["global_prenorm_us_per_call"] = round(pre_us, 2)
    mq_res["global_prenorm_GBps"] = round((sum(gb.values()) + 512 * 4) / (pre_us * 1e-6) / 1e9, 1)
    log(f"global prenorm {pre_us:.1f} us")
    del d_pw, o_pw
    # the global call on an fp32 K=V cache: the workload's bf16 values widened
    # on the device (tiled [P][1][64][16][8] -> [P][1][128][16][4])
    P = d_gl[1].shape[0]
    kv32 = d_gl[1].float().view(P, 1, 64, 16, 2, 4).permute(0, 1, 2, 4, 3, 5).reshape(P, 1, 128, 16, 4).contiguous()
    q32 = d_gl[0].float()
    o32 = torch.empty((64, 16, 512), dtype=torch.float32, device="cuda")
    f32_us = time_calls(lambda: da.attn_decode_global(q32, kv32, *d_gl[2:4], out=o32, num_splits=num_splits),
                        n_extra)
    mq_res["global_f32kv_us_per_call"] = round(f32_us, 2)
    mq_res["global_f32kv_GBps"] = round((2 * (gb["kv"] + gb["q"]) + gb["out"] + gb["table"]) / (f32_us * 1e-6) / 1e9,
                                        1)
    log(f"global fp32 KV {f32_us:.1f} us")
    del kv32, q32, o32
    gate_b = 64 * 16 * 4
    extra = {**mq_res,
        "append_sliding_us_per_call": round(app_sl_us, 2),
        "append_sliding_GBps": round(append_bytes(aws) / (app_sl_us * 1e-6) / 1e9, 1),
        "append_global_us_per_call": round(app_gl_us, 2),
        "append_global_GBps": round(append_bytes(awg) / (app_gl_us * 1e-6) / 1e9, 1),
        "append_calls": "bound (da.bind: Python-side checks once, then the C call alone)",
        "append_sliding_checked_us_per_call": round(app_sl_checked_us, 2),
        "append_global_checked_us_per_call": round(app_gl_checked_us, 2),
        "sliding_gated_us_per_call": round(gsl_us, 2),
        "sliding_gated_GBps": round((sum(sb.values()) + gate_b * 256) / (gsl_us * 1e-6) / 1e9, 1),
        "global_gated_us_per_call": round(ggl_us, 2),
        "global_gated_GBps": round((sum(gb.values()) + gate_b * 512) / (ggl_us * 1e-6) / 1e9, 1),
    }
    log(f"append sliding {app_sl_us:.1f} us ({app_sl_checked_us:.1f} checked), append global {app_gl_us:.1f} us "
        f"({app_gl_checked_us:.1f} checked), "
        f"gated sliding {gsl_us:.1f} us, gated global {ggl_us:.1f} us")

    return extra


def time_sweep(da, I, n_steps, oracle_threads, cpu_out):
    """The full decode step of the model: 48 layer calls (layer i global iff
    i % 6 == 5) at B = 256, lengths log-uniform in [1, 131072], every layer
    with its own caches (drawn on the device). Timed after the B = 64 step,
    not part of it."""
    import types
    import numpy as np
    import torch
    sl = I.sweep_seq_lens()
    t = time.perf_counter()
    layers = []
    for i in range(I.SWEEP["layers"]):
        layers.append(I.device_layer(I.sweep_kind(i), sl, layer=i))
    torch.cuda.synchronize()
    log(f"sweep: 48 layers drawn on the device in {time.perf_counter() - t:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated)")
    outs = {k: torch.empty((len(sl), 16, d), dtype=torch.float32, device="cuda")
            for k, d in (("sliding", 256), ("global", 512))}

    def call(dl):
        if dl.kind == "sliding":
            da.attn_decode_sliding(dl.q, *dl.caches, dl.block_table, dl.seq_lens, dl.window, out=outs["sliding"])
        else:
            da.attn_decode_global(dl.q, *dl.caches, dl.block_table, dl.seq_lens, out=outs["global"])

    def wl(dl):
        lens = dl.host_seq_lens if hasattr(dl, "host_seq_lens") else dl.seq_lens
        return types.SimpleNamespace(seq_lens=lens, window=getattr(dl, "window", 0), kv_dtype="bf16",
                                     Hkv=dl.Hkv, G=dl.G, D=dl.D)

    nbytes = {k: 0 for k in ("sliding", "global")}
    for dl in layers:
        f = sliding_bytes if dl.kind == "sliding" else global_bytes
        nbytes[dl.kind] += sum(f(wl(dl)).values())
    for dl in layers:  # warm-up step
        call(dl)
    torch.cuda.synchronize()
    # per-call event times over one step
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in layers]
    for dl, (e0, e1) in zip(layers, ev):
        e0.record()
        call(dl)
        e1.record()
    torch.cuda.synchronize()
    us = {k: [] for k in ("sliding", "global")}
    for dl, (e0, e1) in zip(layers, ev):
        us[dl.kind].append(e0.elapsed_time(e1) * 1e3)
    # whole steps back to back
    t0 = time.perf_counter()
    for _ in range(n_steps):
        for dl in layers:
            call(dl)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) / n_steps * 1e3
    total = nbytes["sliding"] + nbytes["global"]
    res = {
        "sweep_workload": "48 layer calls (8 global D=512 K=V, 40 sliding D=256 w=1024), B=256, "
                          "seq_lens log-uniform [1,131072], own caches per layer",
        "sweep_ms_per_step": round(step_ms, 3),
        "sweep_bytes_per_step": int(total),
        "sweep_GBps": round(total / (step_ms * 1e-3) / 1e9, 1),
        "sweep_frac_of_peak": round(total / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "sweep_sliding_us_per_call": round(float(np.mean(us["sliding"])), 2),
        "sweep_global_us_per_call": round(float(np.mean(us["global"])), 2),
        "sweep_sliding_GBps": round(nbytes["sliding"] / 40 / (np.mean(us["sliding"]) * 1e-6) / 1e9, 1),
        "sweep_global_GBps": round(nbytes["global"] / 8 / (np.mean(us["global"]) * 1e-6) / 1e9, 1),
    }
    log("sweep: " + ", ".join(f"{k}={v}" for k, v in res.items() if k != "sweep_workload"))
    if oracle_threads > 0:
        # the oracle on a seeded sample of 4 sequences through all 48 layers
        # (stored bytes copied back), extrapolated to the whole step by bytes
        rows = np.sort(np.random.default_rng(4).choice(len(sl), 4, replace=False))
        t_s, b_s = 0.0, 0
        for dl in layers:
            h = I.sample_to_host(dl, rows)
            fn = oracle_sliding_fn(h) if dl.kind == "sliding" else oracle_global_fn(h)
            t_s += time_oracle_rows(fn, range(len(rows)), oracle_threads)
            b_s += sum((sliding_bytes if dl.kind == "sliding" else global_bytes)(wl(h)).values())
            del h
        rate = b_s / t_s
        cpu_out["full_step_48_calls_B256"] = {
            "seconds_sampled": round(t_s, 3), "GBps": round(rate / 1e9, 4),
            "seconds_per_step_extrapolated": round(total / rate, 1),
            "sample": (f"sampled: sequences {rows.tolist()} of 256 (lengths "
                       f"{sl[rows].tolist()}) through all 48 layers, 4 threads; rate extrapolated to the "
                       f"whole step by algorithmic bytes")}
        log(f"oracle: sweep sample {t_s:.1f} s, {rate / 1e9:.3f} GB/s")
    del layers, outs
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing on the host")
    ap.add_argument("--num-splits", type=int, default=0, help="global kernel workgroups (0 = auto)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, copy this many MiB device-to-device once, so that a "
                         "counter profile holds a plain copy of known size to scale HBM counters")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP graph replay of the step reported beside the timed eager steps")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 48-call full-step sweep at B = 256 (its caches take ~80 GB of HBM)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip everything timed after the step (appends, gated and multi-query calls, "
                         "HBM probe, cold-cache and long-context timings), so that a kernel trace holds "
                         "the step's dispatches only")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import decode_attention_amd as da
    from workloads import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if not os.path.exists(da.library_path()):
        from decode_attention_amd.build import build
        build()
    da.load_library()

    log("generating config 1 (sliding) and config 2 (global) inputs on the host")
    t = time.perf_counter()
    sl = I.config_workload(1)
    gl = I.config_workload(2)
    log(f"generated in {time.perf_counter() - t:.1f} s; copying to HBM")
    d_sl = [to_dev(x) for x in (sl.q, sl.k_cache, sl.v_cache, sl.block_table, sl.seq_lens)]
    d_gl = [to_dev(x) for x in (gl.q, gl.kv_cache, gl.block_table, gl.seq_lens)]
    out_sl = torch.empty((64, 16, 256), dtype=torch.float32, device="cuda")
    out_gl = torch.empty((64, 16, 512), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step():
        da.attn_decode_sliding(*d_sl[:5], sl.window, out=out_sl)
        da.attn_decode_global(*d_gl, out=out_gl, num_splits=args.num_splits)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")

    # Per-call times: K steps with HIP events around each call (on torch's
    # current stream, the one the binding passes to the library).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        e[0].record()
        da.attn_decode_sliding(*d_sl[:5], sl.window, out=out_sl)
        e[1].record()
        da.attn_decode_global(*d_gl, out=out_gl, num_splits=args.num_splits)
        e[2].record()
    torch.cuda.synchronize()
    ev_wall = time.perf_counter() - t0
    sl_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    gl_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    sl_med = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    gl_med = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    log(f"per call: sliding {sl_ms * 1e3:.1f} us, global {gl_ms * 1e3:.1f} us "
        f"({ev_wall / args.steps * 1e3:.3f} ms/step with the events)")

    # The timed region: exactly K steps of eager calls, nothing else queued
    # between them, bracketed by device synchronisation.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed: {args.steps} steps, {wall / args.steps * 1e3:.3f} ms/step")

    sb, gb = sliding_bytes(sl), global_bytes(gl)
    step_bytes = sum(sb.values()) + sum(gb.values())
    eager_ms = wall / args.steps * 1e3
    ms_per_step, graph_ms = eager_ms, None
    if not args.no_graph:
        # Context: the same step captured once into a HIP graph and replayed K
        # times (each replay is one graph launch; the runtime leaves ~10 us
        # between replays). Warm-up on the capture's side stream first (the
        # library's workspace is cached per stream).
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) / args.steps * 1e3
        log(f"graph replay: {graph_ms * 1e3:.1f} us/step (eager {eager_ms * 1e3:.1f})")
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    g_ach = sum(gb.values()) / (gl_ms * 1e-3) / 1e9
    s_ach = sum(sb.values()) / (sl_ms * 1e-3) / 1e9

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration_mib} MiB device-to-device for counter calibration")
        del src, dst

    threads = oracle_workers() if not args.no_cpu_baseline else 0
    cpu_more = {}
    extra = {} if args.no_extras else time_extras(da, I, sl, gl, d_sl, d_gl, out_sl, out_gl, sb, gb,
                                                  max(args.steps, 10), args.num_splits)
    if not args.no_extras:
        extra.update(time_context(da, I, sl, gl, d_sl, d_gl, out_sl, out_gl, sb, gb, args.num_splits,
                                  threads, cpu_more))
    if not (args.no_extras or args.no_sweep):
        extra.update(time_sweep(da, I, 5, threads, cpu_more))

    current = counters_current() and args.num_splits == 0  # counters taken at the default split
    traffic = GLOBAL_TRAFFIC["bytes_per_call"] if current else None
    cpu = None
    if threads > 0:
        log(f"timing the oracle on the step's workload ({threads} threads)")
        cpu = cpu_baseline(sl, gl, threads)
        cpu["workloads"].update(cpu_more)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("gemma4-12b decode attention, B=64, seq_lens U[1,32768]: one sliding-layer call "
                         "(Hkv=8, G=2, D=256, window 1024) + one global-layer call (Hkv=1, G=16, D=512, K=V)"),
            "global_batch": 64,
            "seq_len": "U[1,32768]",
            "parallelism": "single GPU",
            "step_timing": "K eager steps, no events in the timed region",
            "graph_replay_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
            "events_ms_per_step": round(ev_wall / args.steps * 1e3, 4),
            "sliding_us_per_call": round(sl_ms * 1e3, 2),
            "global_us_per_call": round(gl_ms * 1e3, 2),
            "sliding_us_median": round(sl_med * 1e3, 2),
            "global_us_median": round(gl_med * 1e3, 2),
            "sliding_GBps": round(s_ach, 1),
            "global_GBps": round(g_ach, 1),
            "sliding_frac_of_peak": round(s_ach / HBM_PEAK_GBS, 4),
            "global_frac_of_peak": round(g_ach / HBM_PEAK_GBS, 4),
            "bytes_per_step": step_bytes,
            "num_splits": args.num_splits,
            "global_algorithmic_bytes_per_call": sum(gb.values()),
            "global_traffic_over_algorithmic": (round(traffic / sum(gb.values()), 4)
                                                if traffic is not None else None),
            "global_mfma_busy": GLOBAL_TRAFFIC["mfma_busy"] if current else None,
            **extra,
        },
        "roofline": {
            "kernel": "attn_decode_global (global_decode_kernel + lse_merge_kernel)",
            "bound": "hbm",
            "achieved": round(g_ach, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(g_ach / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "timing": ("event-timed: HIP events on the library's stream around each attn_decode_global call "
                       "of K steps (both kernels of the call, plus the dispatch gap after the preceding "
                       "sliding call); algorithmic bytes of the call / mean event time"),
            "traffic_source": (None if traffic is None else
                               "FETCH_SIZE x2 + WRITE_SIZE x1 per call from rocprofv3 --pmc passes, "
                               "profiles/decode_attn_B64_seqU1-32768_hbm_counters.md"),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
