"""GPU parity of attn_decode_global (values = keys, split over workgroups with
the log-sum-exp merge) against the fp64 oracle, through the C ABI.

Bar: max-abs 2e-2 for bf16 KV (fp32 accumulate, fp32 out).
"""

import numpy as np
import pytest

import oracle
from workloads import inputs as I

from gpu_util import BF16_TOL, dev, global_on_gpu, max_abs, oracle_rows_parallel

pytestmark = pytest.mark.gpu


def oracle_rows(wl, rows):
    sub_q = wl.q[rows]
    return oracle.paged_decode_global(sub_q, wl.kv_cache, wl.block_table[rows], wl.seq_lens[rows],
                                      wl.kv_dtype)


def check(wl, label, num_splits=0, rows=None):
    print(f"[global] {label}: B={len(wl.seq_lens)} splits={num_splits}", flush=True)
    got = global_on_gpu(wl, num_splits)
    rows = np.arange(len(wl.seq_lens)) if rows is None else np.asarray(rows)
    ref = oracle_rows(wl, rows)
    err = max_abs(got[rows], ref)
    print(f"[global] {label}: max-abs error {err:.3e} over {len(rows)} sequences", flush=True)
    assert np.isfinite(got).all(), label
    assert err <= BF16_TOL, (label, err)
    return got, ref


SMALL = [0, 1, 2, 15, 16, 17, 100, 1000, 4097, 333]


# (with B = 10, splits 2-64 take the merge's two-group form, 100 its
# four-group form, 0 (256) its quarter-tile form and 1000 the wide one)
@pytest.mark.parametrize("num_splits", [0, 1, 2, 3, 7, 64, 100, 1000])
def test_ragged_lengths_every_split(gpu_lib, num_splits):
    wl = I.make_global(SMALL, kv_dtype="bf16", tag=(400,), **I.GLOBAL)
    got, _ = check(wl, "ragged", num_splits)
    assert np.all(got[0] == 0)


@pytest.mark.parametrize("num_splits", [0, 1, 3, 17, 100])
def test_many_short_sequences(gpu_lib, num_splits):
    # 1-3 pages per sequence: two-page steps often straddle a sequence start,
    # and workgroup ranges cut sequences at odd page offsets.
    rng = np.random.default_rng(405)
    lens = rng.integers(1, 48, size=200)
    wl = I.make_global(lens, kv_dtype="bf16", tag=(405,), **I.GLOBAL)
    check(wl, f"short sequences, splits {num_splits}", num_splits)


@pytest.mark.parametrize("num_splits", [0, 250, 2500, 9000])
def test_short_and_empty_sequences_weighted_split(gpu_lib, num_splits):
    # The split weighs each non-empty sequence start as 8 pages. With 1-3
    # page sequences most workgroup ranges hold only such weight and no page
    # (0, 250); past the weighted total (1787 here: 2500, 9000) many ranges
    # are empty as well. Empty sequences carry no weight and get zero rows.
    rng = np.random.default_rng(406)
    lens = rng.integers(1, 41, size=256)
    lens[rng.random(256) < 0.25] = 0
    wl = I.make_global(lens, kv_dtype="bf16", tag=(406,), **I.GLOBAL)
    got, _ = check(wl, f"short and empty sequences, splits {num_splits}", num_splits)
    assert np.all(got[lens == 0] == 0)


def test_split_invariance(gpu_lib):
    wl = I.make_global([5000, 1, 20000, 7777], kv_dtype="bf16", tag=(401,), **I.GLOBAL)
    outs = [global_on_gpu(wl, s) for s in (1, 2, 5, 37, 256, 0)]
    # The weights reach the MFMAs as bf16 hi + lo parts (about 2^-17 relative),
    # so splits differ only by that and by fp32 summation order.
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= 2e-4
    ref = oracle_rows(wl, np.arange(4))
    assert max_abs(outs[0], ref) <= BF16_TOL


def test_single_token_returns_its_row(gpu_lib):
    wl = I.make_global([1, 1, 1], kv_dtype="bf16", tag=(402,), **I.GLOBAL)
    got = global_on_gpu(wl)
    for b in range(3):
        k = oracle.gather_tiled_cache(wl.kv_cache, wl.block_table[b], [0])[0, 0]
        kf = oracle.stored_to_f64(k, "bf16")
        np.testing.assert_array_equal(got[b], np.broadcast_to(kf, (16, 512)))


@pytest.mark.parametrize("mode", ["q_zero", "q_small"])
def test_diffuse_softmax(gpu_lib, mode):
    kw = dict(q_zero=True) if mode == "q_zero" else dict(q_scale=1 / 22.6)
    wl = I.make_global([1, 300, 5000], kv_dtype="bf16", tag=(403,), **I.GLOBAL, **kw)
    check(wl, mode)


def test_deterministic(gpu_lib):
    wl = I.make_global([10000, 3, 777], kv_dtype="bf16", tag=(404,), **I.GLOBAL)
    for splits in (0, 37, 256):
        assert np.array_equal(global_on_gpu(wl, splits), global_on_gpu(wl, splits))


@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_empty_sequences_are_written(gpu_lib, num_splits):
    # Rows of sequences without cached tokens are zero even where the output
    # buffer held NaN, whatever the split.
    import torch
    import decode_attention_amd as da
    wl = I.make_global([0, 40, 0, 3000, 0], kv_dtype="bf16", tag=(407,), **I.GLOBAL)
    q, kv, bt, sl = (dev(x) for x in (wl.q, wl.kv_cache, wl.block_table, wl.seq_lens))
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device="cuda")
    da.attn_decode_global(q, kv, bt, sl, out=out, num_splits=num_splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(got[[0, 2, 4]] == 0)
    assert max_abs(got[[1, 3]], oracle_rows(wl, [1, 3])) <= BF16_TOL


def test_config2_full_size_every_row(gpu_lib):
    wl = I.config_workload(2)
    print(f"[global] config 2: B=64 splits=0", flush=True)
    got = global_on_gpu(wl)
    ref = oracle_rows_parallel(lambda b: oracle_rows(wl, [b])[0], range(64))
    err = max_abs(got, ref)
    print(f"[global] config 2: max-abs error {err:.3e} over 64 of 64 sequences", flush=True)
    assert np.isfinite(got).all()
    assert err <= BF16_TOL


def test_config3_long_context(gpu_lib):
    wl = I.config_workload(3)
    check(wl, "config 3")


@pytest.mark.parametrize("num_splits", [0, 5])
def test_page_permutation_invariant_and_read_only(gpu_lib, num_splits):
    """Re-placing the pages (block table updated to match) gives the same
    output bit for bit, and the call leaves the cache as it found it."""
    import torch

    import decode_attention_amd as da
    a = I.make_global([1, 300, 5000, 16, 2049, 777], kv_dtype="bf16", tag=(230,), **I.GLOBAL)
    q, kv = dev(a.q), dev(a.kv_cache)
    bt, sl = dev(a.block_table), dev(a.seq_lens)
    ksum = kv.view(torch.int16).to(torch.int64).sum().item()
    o1 = da.attn_decode_global(q, kv, bt, sl, num_splits=num_splits).cpu()
    torch.cuda.synchronize()
    assert kv.view(torch.int16).to(torch.int64).sum().item() == ksum
    guard = a.meta["num_pages"] - 1
    perm = np.random.default_rng(8).permutation(guard)
    kv2 = a.kv_cache.copy()
    kv2[perm] = a.kv_cache[:-1]
    bt2 = a.block_table.copy()
    used = bt2 != guard
    bt2[used] = perm[bt2[used]]
    print(f"[global] permuted placement: splits={num_splits} pages={guard}", flush=True)
    o2 = da.attn_decode_global(q, dev(kv2), dev(bt2), sl, num_splits=num_splits).cpu()
    assert torch.equal(o1, o2)
