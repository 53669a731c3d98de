"""Runs one benchmark workload's call a number of times, for an external
profiler (measurement support, not part of the attention path):

    python -m workloads.profile_run WORKLOAD [--iters N]

after one untimed call, N calls back to back on the library's stream, then
the mean time per call by HIP events. The workloads are the ones the
benchmark times, built by the same seeded generators:

  global_b64          global layer, B = 64, lengths uniform in [1, 32768]
  sliding_b64         sliding layer (window 1024), the same lengths
  long_context        global layer, B = 2, lengths 131072 and 262144
  global_sweep_b256   one global layer of the 48-call step sweep (layer 5),
                        B = 256, lengths log-uniform in [1, 131072]
  prenorm_b64         global layer from the pre-norm projection, B = 64
  global_b64_f32      global layer, B = 64, the same lengths, fp32 K=V cache
                        (global_b64's bf16 values widened on the device)
  mq_verify_global    8 queries per sequence (speculative verification),
  mq_verify_sliding     B = 64, the decode workloads' lengths
  mq_prefill_global   one 2048-token prefill chunk per sequence, B = 4
  mq_prefill_sliding    (length 8192 global, 4096 sliding)
"""

import argparse
import sys

import numpy as np

WORKLOADS = ("global_b64", "sliding_b64", "long_context", "global_sweep_b256", "prenorm_b64", "global_b64_f32",
             "mq_verify_global",
             "mq_verify_sliding", "mq_prefill_global", "mq_prefill_sliding")


def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def build_call(name):
    """Returns a zero-argument callable making the workload's call once."""
    import torch
    import decode_attention_amd as da
    from . import inputs as I
    if name in ("global_b64", "sliding_b64", "prenorm_b64", "global_b64_f32") or name.startswith("mq_"):
        sl, gl = I.config_workload(1), I.config_workload(2)
    if name == "global_b64":
        args = [_dev(x) for x in (gl.q, gl.kv_cache, gl.block_table, gl.seq_lens)]
        out = torch.empty((64, 16, 512), dtype=torch.float32, device="cuda")
        return lambda: da.attn_decode_global(*args, out=out)
    if name == "global_b64_f32":
        q, kv, bt, sl = (_dev(x) for x in (gl.q, gl.kv_cache, gl.block_table, gl.seq_lens))
        P = kv.shape[0]
        # tiled bf16 [P][1][64][16][8] -> tiled fp32 [P][1][128][16][4]: chunk c
        # of 8 coordinates becomes chunks 2c and 2c + 1 of 4
        kv32 = kv.float().view(P, 1, 64, 16, 2, 4).permute(0, 1, 2, 4, 3, 5).reshape(P, 1, 128, 16, 4).contiguous()
        del kv
        q32 = q.float()
        out = torch.empty((64, 16, 512), dtype=torch.float32, device="cuda")
        return lambda: da.attn_decode_global(q32, kv32, bt, sl, out=out)
    if name == "sliding_b64":
        args = [_dev(x) for x in (sl.q, sl.k_cache, sl.v_cache, sl.block_table, sl.seq_lens)]
        out = torch.empty((64, 16, 256), dtype=torch.float32, device="cuda")
        return lambda: da.attn_decode_sliding(*args, sl.window, out=out)
    if name == "long_context":
        dl = I.device_layer("global", [131072, 262144], tag=(3,))
        out = torch.empty((2, 16, 512), dtype=torch.float32, device="cuda")
        return lambda: da.attn_decode_global(dl.q, *dl.caches, dl.block_table, dl.seq_lens, out=out)
    if name == "global_sweep_b256":
        dl = I.device_layer("global", I.sweep_seq_lens(), layer=5)
        out = torch.empty((I.SWEEP["B"], 16, 512), dtype=torch.float32, device="cuda")
        return lambda: da.attn_decode_global(dl.q, *dl.caches, dl.block_table, dl.seq_lens, out=out)
    if name == "prenorm_b64":
        pw = I.make_global_prenorm(gl.seq_lens, tag=(708,), P_max=2048)
        args = [_dev(x) for x in (pw.q, pw.x_cache, pw.w_k, pw.block_table, pw.seq_lens)]
        out = torch.empty((64, 16, 512), dtype=torch.float32, device="cuda")
        return lambda: da.attn_decode_global_prenorm(*args, out=out)
    shp = dict(Hkv=sl.Hkv, G=sl.G, D=sl.D)
    if name == "mq_verify_sliding":
        mq = I.make_multiquery("sliding", sl.seq_lens, np.full(64, 8), tag=(704,), P_max=2048, **shp,
                               window=sl.window)
    elif name == "mq_verify_global":
        q8 = I.rms_rows(I.rng_for((705,), 0, I.STREAM_MQ), (64 * 8, gl.Hkv * gl.G, gl.D))
        mq = I.MultiQueryWorkload("global", I.to_storage(q8, "bf16"), np.arange(0, 65 * 8, 8, dtype=np.int32), gl)
    elif name == "mq_prefill_sliding":
        mq = I.make_multiquery("sliding", [4096] * 4, [2048] * 4, tag=(706,), **shp, window=sl.window)
    elif name == "mq_prefill_global":
        mq = I.make_multiquery("global", [8192] * 4, [2048] * 4, tag=(707,), **I.GLOBAL)
    else:
        raise ValueError(f"unknown workload {name!r}; one of {', '.join(WORKLOADS)}")
    base = mq.base
    args = [_dev(mq.q), _dev(mq.q_start), mq.max_queries]
    tail = [_dev(base.block_table), _dev(base.seq_lens)]
    out = torch.empty(mq.q.shape, dtype=torch.float32, device="cuda")
    if mq.kind == "sliding":
        caches = [_dev(base.k_cache), _dev(base.v_cache)]
        return lambda: da.attn_multiquery_sliding(*args, *caches, *tail, base.window, out=out)
    cache = _dev(base.kv_cache)
    return lambda: da.attn_multiquery_global(*args, cache, *tail, out=out)


def main(argv=None):
    import torch
    ap = argparse.ArgumentParser(description="run one benchmark workload's call N times (for a profiler)")
    ap.add_argument("workload", choices=WORKLOADS)
    ap.add_argument("--iters", type=int, default=10)
    args = ap.parse_args(argv)
    torch.cuda.set_device(0)
    fn = build_call(args.workload)
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    print(f"{args.workload}: {args.iters} calls, {e0.elapsed_time(e1) * 1e3 / max(args.iters, 1):.1f} us per call "
          "(HIP events)", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
