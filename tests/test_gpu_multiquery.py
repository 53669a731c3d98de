"""GPU parity of attn_multiquery_sliding / attn_multiquery_global (several
queries per sequence at its last positions: chunked prefill, speculative
verification) against the fp64 oracle, through the C ABI.

Bar: max-abs 2e-2 (bf16 KV, fp32 accumulate and output). At full sizes the
oracle checks sampled query rows one by one through the decode oracle on the
sequence cut to the row's position + 1, which is the same quantity.
"""

import numpy as np
import pytest
import torch

import decode_attention_amd as da
import oracle
from workloads import inputs as I

from gpu_util import BF16_TOL, dev, max_abs

pytestmark = pytest.mark.gpu


def run(mq, num_splits=0):
    base = mq.base
    q, qs = dev(mq.q), dev(mq.q_start)
    bt, sl = dev(base.block_table), dev(base.seq_lens)
    if mq.kind == "sliding":
        o = da.attn_multiquery_sliding(q, qs, max(mq.max_queries, 1), dev(base.k_cache), dev(base.v_cache), bt, sl,
                                       base.window, num_splits=num_splits)
    else:
        o = da.attn_multiquery_global(q, qs, max(mq.max_queries, 1), dev(base.kv_cache), bt, sl,
                                      num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64)


def oracle_all(mq):
    base = mq.base
    if mq.kind == "sliding":
        return oracle.paged_multiquery_sliding(mq.q, mq.q_start, base.k_cache, base.v_cache, base.block_table,
                                               base.seq_lens, base.window, base.kv_dtype)
    return oracle.paged_multiquery_global(mq.q, mq.q_start, base.kv_cache, base.block_table, base.seq_lens,
                                          base.kv_dtype)


def oracle_row(mq, b, j):
    """Query j of sequence b, through the decode oracle on the sequence cut to
    the query's position + 1."""
    base = mq.base
    L, S = int(base.seq_lens[b]), int(mq.q_start[b + 1] - mq.q_start[b])
    pos = L - S + j
    s = int(mq.q_start[b]) + j
    if pos < 0:
        return np.zeros(mq.q.shape[1:])
    q, bt, sl = mq.q[s][None], base.block_table[b][None], np.array([pos + 1], dtype=np.int32)
    if mq.kind == "sliding":
        return oracle.paged_decode_sliding(q, base.k_cache, base.v_cache, bt, sl, base.window, base.kv_dtype)[0]
    return oracle.paged_decode_global(q, base.kv_cache, bt, sl, base.kv_dtype)[0]


def check(mq, label, num_splits=0):
    print(f"[multiquery] {mq.kind} {label}: B={len(mq.base.seq_lens)} T={mq.q.shape[0]} splits={num_splits}",
          flush=True)
    got = run(mq, num_splits)
    err = max_abs(got, oracle_all(mq))
    print(f"[multiquery] {mq.kind} {label}: max-abs error {err:.3e}", flush=True)
    assert np.isfinite(got).all(), label
    assert err <= BF16_TOL, (label, err)
    return got


SL_LENS = [1, 16, 17, 40, 300, 1100, 2100, 64]
SL_COUNTS = [1, 3, 17, 40, 64, 65, 130, 64]


@pytest.mark.parametrize("num_splits", [0, 1, 2, 5])
def test_sliding_ragged(gpu_lib, num_splits):
    mq = I.make_multiquery("sliding", SL_LENS, SL_COUNTS, tag=(900,), **I.SLIDING)
    check(mq, "ragged", num_splits)


@pytest.mark.parametrize("window", [1, 7, 16, 100])
def test_sliding_windows(gpu_lib, window):
    mq = I.make_multiquery("sliding", [5, 33, 200, 700], [5, 20, 70, 9], tag=(901, window), Hkv=8, G=2, D=256,
                           window=window)
    check(mq, f"window {window}")


GL_LENS = [1, 5, 17, 100, 1000, 5000, 33]
GL_COUNTS = [1, 2, 4, 5, 9, 33, 33]


@pytest.mark.parametrize("num_splits", [0, 1, 3, 8])
def test_global_ragged(gpu_lib, num_splits):
    mq = I.make_multiquery("global", GL_LENS, GL_COUNTS, tag=(902,), **I.GLOBAL)
    check(mq, "ragged", num_splits)


@pytest.mark.parametrize("kind", ["sliding", "global"])
def test_more_queries_than_keys_and_empty_sequences(gpu_lib, kind):
    shape = I.SLIDING if kind == "sliding" else I.GLOBAL
    mq = I.make_multiquery(kind, [3, 0, 20, 9], [7, 0, 20, 2], tag=(903,), **shape)
    got = check(mq, "S > L")
    assert np.all(got[:4] == 0)  # positions -4 .. -1 see nothing


@pytest.mark.parametrize("kind", ["sliding", "global"])
def test_deterministic(gpu_lib, kind):
    shape = I.SLIDING if kind == "sliding" else I.GLOBAL
    mq = I.make_multiquery(kind, [3000, 700], [40, 9], tag=(904,), **shape)
    for splits in (0, 3):
        assert np.array_equal(run(mq, splits), run(mq, splits))


def test_split_invariance_global(gpu_lib):
    # Each piece rounds its weights to bf16 against its own reference, so
    # results of different splits differ by that rounding (2^-9 relative per
    # weight), not by fp32 order alone; a wrong merge would be off by O(1).
    mq = I.make_multiquery("global", [6000, 20], [12, 12], tag=(905,), **I.GLOBAL)
    ref = oracle_all(mq)
    outs = [run(mq, s) for s in (1, 2, 7, 30)]
    for o in outs:
        assert max_abs(o, ref) <= BF16_TOL
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= BF16_TOL


@pytest.mark.parametrize("kind", ["sliding", "global"])
@pytest.mark.parametrize("q_scale", [0.3, 0.05])
def test_diffuse_softmax(gpu_lib, kind, q_scale):
    shape = I.SLIDING if kind == "sliding" else I.GLOBAL
    mq = I.make_multiquery(kind, [2000, 5000, 77], [64, 5, 30], tag=(909,), q_scale=q_scale, **shape)
    check(mq, f"q scale {q_scale}", 0)
    check(mq, f"q scale {q_scale}", 3)


def sampled_check(mq, label, picks):
    print(f"[multiquery] {mq.kind} {label}: B={len(mq.base.seq_lens)} T={mq.q.shape[0]}", flush=True)
    got = run(mq)
    assert np.isfinite(got).all()
    err = 0.0
    for b, j in picks:
        err = max(err, max_abs(got[int(mq.q_start[b]) + j], oracle_row(mq, b, j)))
    print(f"[multiquery] {mq.kind} {label}: max-abs error {err:.3e} over {len(picks)} sampled rows", flush=True)
    assert err <= BF16_TOL, (label, err)


def test_speculative_verify_global_B64(gpu_lib):
    # 8 draft tokens per sequence at the global decode workload's lengths
    sl = I.uniform_seq_lens((2,), 64, 8, 32768)
    mq = I.make_multiquery("global", sl, np.full(64, 8), tag=(906,), P_max=2048, **I.GLOBAL)
    order = np.argsort(sl)
    picks = [(int(b), j) for b in np.concatenate([order[:2], order[-2:], [5]]) for j in (0, 3, 7)]
    sampled_check(mq, "verify B=64 S=8", picks)


def test_speculative_verify_sliding_B64(gpu_lib):
    sl = I.uniform_seq_lens((1,), 64, 8, 32768)
    mq = I.make_multiquery("sliding", sl, np.full(64, 8), tag=(907,), P_max=2048, **I.SLIDING)
    picks = [(int(b), j) for b in (0, 17, 40, 63) for j in (0, 7)]
    sampled_check(mq, "verify B=64 S=8", picks)


@pytest.mark.parametrize("kind", ["sliding", "global"])
def test_chunked_prefill(gpu_lib, kind):
    # one 2048-token chunk appended to 2048 (sliding) or 6144 (global) earlier tokens
    shape = I.SLIDING if kind == "sliding" else I.GLOBAL
    L = 4096 if kind == "sliding" else 8192
    mq = I.make_multiquery(kind, [L, 1500], [2048, 300], tag=(908,), **shape)
    picks = [(0, j) for j in (0, 1, 63, 64, 1000, 1023, 1024, 1025, 2047)] + [(1, j) for j in (0, 150, 299)]
    sampled_check(mq, "prefill chunk 2048", picks)


def test_balanced_split_one_long_sequence(gpu_lib):
    # Speculative verification where one sequence holds almost every page:
    # the default split gives that sequence's row blocks most of the grid
    # (hundreds of pieces each, folded by the merge) and the short ones one
    # piece each.
    lens = np.concatenate([[100000], np.arange(1, 64) * 5])
    mq = I.make_multiquery("global", lens, np.full(64, 8), tag=(910,), **I.GLOBAL)
    got = run(mq)
    assert np.isfinite(got).all()
    for b, j in [(0, 0), (0, 7), (1, 0), (33, 5), (63, 7)]:
        s = int(mq.q_start[b]) + j
        err = max_abs(got[s], oracle_row(mq, b, j))
        print(f"[multiquery] one long sequence: b={b} query {j}: max-abs {err:.3e}", flush=True)
        assert err <= BF16_TOL


def test_contiguous_split_short_units(gpu_lib):
    # The global layers' default split lays the steps of all row blocks end
    # to end and gives each workgroup an equal share: here most shares hold
    # many short blocks whole (written directly), blocks cut by a share
    # boundary go through the merge, and blocks with queries but no cached
    # key (L = 0) or no queries at all are met by no workgroup.
    rng = np.random.default_rng(911)
    lens = rng.integers(0, 90, size=300)
    counts = np.minimum(rng.integers(0, 13, size=300), np.maximum(lens, 1))
    counts[5::23] = 0
    lens[::17] = 0
    counts[::17] = 3  # queries at positions -3 .. -1: all-zero rows
    lens[7] = 40000  # one block longer than a share
    counts[7] = 8
    mq = I.make_multiquery("global", lens, counts, tag=(911,), **I.GLOBAL)
    got = check(mq, "contiguous split, short units")
    for b in range(0, 300, 17):
        s = int(mq.q_start[b])
        assert np.all(got[s:s + 3] == 0)
    assert np.array_equal(got, run(mq))


@pytest.mark.parametrize("window,num_splits", [(0, 0), (1, 3), (17, 0), (100, 3), (1024, 0), (1024, 3), (4096, 0)])
def test_long_sliding_chunks_windows(gpu_lib, window, num_splits):
    # 128 queries or more in a sequence: the sliding layers' 32-row-tile
    # kernel (256-row blocks). Ragged chunks with block boundaries inside and
    # at the ends, queries before position 0 (S > L), windows from 0 (all
    # zero) to wider than every sequence, and both splits.
    lens = [300, 128, 2000, 1500, 100, 4096]
    counts = [300, 128, 129, 257, 130, 1]
    mq = I.make_multiquery("sliding", lens, counts, tag=(912, window), Hkv=8, G=2, D=256, window=window)
    got = check(mq, f"long chunks, window {window}", num_splits)
    if window == 0:
        assert np.all(got == 0)
    s = int(mq.q_start[4])
    assert np.all(got[s:s + 30] == 0)  # positions -30 .. -1 see nothing


def test_long_sliding_chunks_whole_blocks(gpu_lib):
    # 8 sequences x 8 KV heads x 8 blocks of 128 queries = 512 blocks, two
    # per compute unit or more: whole blocks, no split or merge
    lens = [3000, 1100, 5000, 1024, 2048, 1500, 4000, 1030]
    mq = I.make_multiquery("sliding", lens, [1024] * 8, tag=(913,), **I.SLIDING)
    picks = [(b, j) for b in range(8) for j in (0, 127, 128, 640, 1023)]
    sampled_check(mq, "long chunks, whole blocks", picks)
