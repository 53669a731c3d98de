"""bench.py on the CPU: its one-GPU contract and the algorithmic byte counts
its GB/s figures and roofline are computed from.

The byte counts are checked against values derived by hand from the
workload definitions (KV read once per visible key, K = V counted once on
global layers, q in the cache dtype, fp32 out, one block-table entry per page
touched plus one sequence length per sequence), not against a retyped copy of
bench.py's formulas.
"""

import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import inputs as I  # noqa: E402


def _wl(seq_lens, **kw):
    return types.SimpleNamespace(seq_lens=np.asarray(seq_lens, np.int32), **kw)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_sliding_bytes_small_case_by_hand():
    # Lengths 1, 17, 1024, 2048 with window 1024, bf16, Hkv 8, D 256:
    # visible keys 1 + 17 + 1024 + 1024; each key is one k and one v row of
    # 256 bf16 per KV head.
    wl = _wl([1, 17, 1024, 2048], window=1024, kv_dtype="bf16", Hkv=8, G=2, D=256)
    b = bench.sliding_bytes(wl)
    assert b["kv"] == (1 + 17 + 1024 + 1024) * 8 * 256 * 2 * 2
    assert b["q"] == 4 * 16 * 256 * 2
    assert b["out"] == 4 * 16 * 256 * 4
    # pages touched: [0], [0, 1], pages 0..63, pages 64..127 (positions
    # 1024..2047); plus one length per sequence
    assert b["table"] == (1 + 2 + 64 + 64) * 4 + 4 * 4


def test_sliding_window_cut_mid_page():
    # L = 1030, w = 1024: keys 6..1029 are visible, pages 0..64 are touched.
    wl = _wl([1030], window=1024, kv_dtype="f32", Hkv=8, G=2, D=256)
    b = bench.sliding_bytes(wl)
    assert b["kv"] == 1024 * 8 * 256 * 2 * 4
    assert b["table"] == 65 * 4 + 4


def test_global_bytes_count_k_equal_v_once():
    wl = _wl([1, 16, 17, 0], kv_dtype="bf16", Hkv=1, G=16, D=512)
    b = bench.global_bytes(wl)
    assert b["kv"] == (1 + 16 + 17) * 512 * 2
    assert b["q"] == 4 * 16 * 512 * 2
    assert b["out"] == 4 * 16 * 512 * 4
    assert b["table"] == (1 + 1 + 2 + 0) * 4 + 4 * 4


def test_benchmark_workloads_are_the_seeded_ones():
    # The B = 64 workloads' lengths, and the global call's algorithmic bytes
    # quoted with the measurements (1 144 870 420 B per call).
    sl = I.uniform_seq_lens((1,), 64, 1, 32768)
    gl = I.uniform_seq_lens((2,), 64, 1, 32768)
    assert len(sl) == len(gl) == 64
    assert sl.min() >= 1 and sl.max() <= 32768 and gl.min() >= 1 and gl.max() <= 32768
    g = bench.global_bytes(_wl(gl, kv_dtype="bf16", Hkv=1, G=16, D=512))
    assert sum(g.values()) == 1144870420
    assert int(((gl.astype(np.int64) + 15) // 16).sum()) == 69701  # pages of the global call


def test_cpu_baseline_describes_its_run():
    # Small stand-ins for the step's two workloads: the baseline times every
    # sequence of both, on the threads it reports, and names the CPU.
    sl = I.make_sliding([1, 17, 1030, 40], kv_dtype="bf16", tag=(31,), **I.SLIDING)
    gl = I.make_global([5, 300, 17], kv_dtype="bf16", tag=(32,), **I.GLOBAL)
    res = bench.cpu_baseline(sl, gl, 3)
    assert res["kind"] == "oracle" and res["unit"] == "GB/s" and res["value"] > 0
    assert res["cores"] == 3 and "3 threads" in res["sample"]
    assert isinstance(res["cpu_model"], str) and res["cpu_model"]
    w = res["workloads"]
    assert set(w) == {"tiny_sliding_fp32_B4", "sliding_bf16_B64", "global_bf16_B64"}
    b = sum(bench.sliding_bytes(sl).values()) + sum(bench.global_bytes(gl).values())
    t = w["sliding_bf16_B64"]["seconds"] + w["global_bf16_B64"]["seconds"]
    assert abs(res["value"] - b / t / 1e9) <= 1e-2 * res["value"] + 1e-4
    assert 1 <= bench.oracle_workers() <= 16
