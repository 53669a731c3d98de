"""Per-workgroup timeline of the global decode call on the benchmark's
workloads (measurement support, not part of the attention path):

    python -m workloads.trace_run [--dump FILE.npz]

runs the global layer workload (B = 64, lengths uniform in [1, 32768]) and
the long-context one (B = 2, lengths 131072 and 262144) through
``attn_decode_global_traced`` and prints when the workgroups start, how
their end times spread, per XCC, next to the call's time by HIP events.
"""

import sys

import numpy as np

from decode_attention_amd.trace import format_summary, global_timeline, summarize


def main(argv=None):
    import argparse
    import torch
    ap = argparse.ArgumentParser(description="per-workgroup timeline of the global decode call")
    ap.add_argument("--dump", default=None, help="also save the raw entries of every traced call (.npz)")
    args_cli = ap.parse_args(argv)
    raw = {}

    import decode_attention_amd.binding as B
    from . import inputs as I
    torch.cuda.set_device(0)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    def event_us(fn, n=20):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    gl = I.config_workload(2)
    args = [dev(x) for x in (gl.q, gl.kv_cache, gl.block_table, gl.seq_lens)]
    out = torch.empty((64, 16, 512), dtype=torch.float32, device="cuda")
    pages = int(((gl.seq_lens.astype(np.int64) + 15) // 16).sum())
    us = event_us(lambda: B.attn_decode_global(*args, out=out))
    for rep in range(3):
        _, e = global_timeline(*args, out)
        raw[f"b64_{rep}"] = e
        print(format_summary(f"global B=64 U[1,32768], traced call {rep}", summarize(e), us if rep == 0 else None,
                             pages), flush=True)
    dl = I.device_layer("global", [131072, 262144], tag=(3,))
    out2 = torch.empty((2, 16, 512), dtype=torch.float32, device="cuda")
    largs = [dl.q, dl.caches[0], dl.block_table, dl.seq_lens]
    us = event_us(lambda: B.attn_decode_global(*largs, out=out2))
    for rep in range(2):
        _, e = global_timeline(*largs, out2)
        raw[f"long_{rep}"] = e
        print(format_summary(f"global long context B=2 {{131072, 262144}}, traced call {rep}", summarize(e),
                             us if rep == 0 else None, (131072 + 262144) // 16), flush=True)
    if args_cli.dump:
        np.savez(args_cli.dump, **raw)
    return 0


if __name__ == "__main__":
    sys.exit(main())
