"""C ABI checks that need no GPU: the library loads, exports every function
include/decode_attn.h declares, and host validation returns the documented
status codes before any HIP call."""

import ctypes
import os
import re

import pytest

import decode_attention_amd as da
from decode_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(da.library_path()):
        from decode_attention_amd.build import build
        build()
    return da.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_api():
    assert declared_functions() == sorted(B.EXPORTS)


def declared_prototypes():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = {}
    for m in re.finditer(r"^\s*((?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\([^;]*\))\s*;", text, flags=re.M):
        protos[m.group(2)] = re.sub(r"\s+", " ", m.group(1)).replace("( ", "(").replace(" )", ")")
    return protos


# The hot path's four calls, as this library declares them. Two departures
# from the plain boundary sketch are deliberate (the workspace size comes
# back through a pointer so that the call can report an invalid shape, and
# the split knob counts workgroups over the batch's page list).
PATH_PROTOTYPES = {
    "attn_decode_sliding": "da_status attn_decode_sliding(const void* q, const void* k_cache, const void* v_cache,"
                           " const int32_t* block_table, const int32_t* seq_lens, int32_t window, void* out,"
                           " const da_shape* shape, void* stream)",
    "attn_decode_global": "da_status attn_decode_global(const void* q, const void* kv_cache,"
                          " const int32_t* block_table, const int32_t* seq_lens, void* out,"
                          " const da_shape* shape, void* workspace, size_t workspace_bytes, void* stream)",
    "attn_decode_global_workspace_bytes": "da_status attn_decode_global_workspace_bytes(const da_shape* shape,"
                                          " size_t* bytes)",
    "attn_status_string": "const char* attn_status_string(da_status status)",
}


def test_hot_path_signatures():
    protos = declared_prototypes()
    for name, want in PATH_PROTOTYPES.items():
        assert protos[name] == want, name


def test_shape_struct_matches_the_binding():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct da_shape \{(.*?)\} da_shape;", text, flags=re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+)\s*;", body)
    assert fields == [f for f, _ in B.DaShape._fields_]
    assert len(re.findall(r";", body)) == len(fields)  # every member is an int32_t


def test_trace_header_symbol_is_exported(lib):
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "decode_attn_trace.h")).read(), flags=re.S)
    names = re.findall(r"^\s*\w+\s+(attn_\w+)\s*\(", text, flags=re.M)
    assert names == ["attn_decode_global_traced"]
    assert hasattr(lib, "attn_decode_global_traced")


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        s = da.attn_status_string(code)
        assert s and s != "unknown status"
    assert da.attn_status_string(-99) == "unknown status"


def _shape(**kw):
    base = dict(batch=4, num_kv_heads=8, group=2, head_dim=256, max_pages_per_seq=8, num_pages=32,
                kv_dtype=B.DA_DTYPE_BF16)
    base.update(kw)
    return B.make_shape(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation rejects first
NULL = ctypes.c_void_p(0)


def sliding(lib, shape, window=1024, ptrs=None):
    p = ptrs or [FAKE] * 6
    return lib.attn_decode_sliding(p[0], p[1], p[2], p[3], p[4], window, p[5], ctypes.byref(shape)
                                   if shape is not None else None, NULL)


def test_sliding_validation(lib):
    assert sliding(lib, None) == -1
    assert sliding(lib, _shape(), window=-1) == -1
    assert sliding(lib, _shape(batch=0)) == -1
    assert sliding(lib, _shape(num_pages=0)) == -1
    assert sliding(lib, _shape(kv_dtype=7)) == -1
    assert sliding(lib, _shape(), ptrs=[FAKE, FAKE, NULL, FAKE, FAKE, FAKE]) == -1
    assert sliding(lib, _shape(head_dim=128)) == -2
    assert sliding(lib, _shape(group=4)) == -2
    for ns in (3, 5, 16):  # waves per unit: 0, 1, 2, 4 or 8 only
        assert sliding(lib, _shape(num_splits=ns)) == -2
    assert sliding(lib, _shape(num_splits=8, kv_dtype=B.DA_DTYPE_F32)) == -2  # 8: bf16 only
    s = _shape()
    s.page_size = 32
    assert sliding(lib, s) == -2
    s = _shape()
    s.out_dtype = 7
    assert sliding(lib, s) == -1


def test_bf16_output_is_valid_for_the_decode_calls_only(lib):
    """out_dtype bf16: accepted by the decode calls (which then stop at the
    device check on a host without a GPU), refused by the multi-query calls
    and the appends, whose outputs are fp32 only."""
    s, g = _shape(), _gshape()
    s.out_dtype = B.DA_DTYPE_BF16
    g.out_dtype = B.DA_DTYPE_BF16
    assert sliding(lib, s) == -4
    assert sliding_gated(lib, s) == -4
    assert glob(lib, g) == -4
    assert global_gated(lib, g) == -4
    assert glob_noalloc(lib, g) == -4
    assert mq(lib, s) == -2
    assert mq(lib, g, sliding=False) == -2
    assert append_sliding(lib, s) == -2
    assert append_global(lib, g) == -2
    assert append_prenorm(lib, g) == -2


def _gshape(**kw):
    base = dict(batch=4, num_kv_heads=1, group=16, head_dim=512, max_pages_per_seq=8, num_pages=32,
                kv_dtype=B.DA_DTYPE_BF16)
    base.update(kw)
    return B.make_shape(**base)


def glob(lib, shape, ws=FAKE, ws_bytes=1 << 30, ptrs=None):
    p = ptrs or [FAKE] * 5
    return lib.attn_decode_global(p[0], p[1], p[2], p[3], p[4], ctypes.byref(shape), ws, ws_bytes, NULL)


def test_global_validation(lib):
    assert glob(lib, _gshape(batch=-1)) == -1
    assert glob(lib, _gshape(), ptrs=[FAKE, NULL, FAKE, FAKE, FAKE]) == -1
    assert glob(lib, _gshape(group=8)) == -2
    assert glob(lib, _gshape(batch=5000)) == -2
    # the split's 32-bit page prefix: batch * max_pages_per_seq <= 2^30
    assert glob(lib, _gshape(batch=256, max_pages_per_seq=1 << 23)) == -2


def traced(lib, shape):
    from decode_attention_amd import trace as T
    T._lib()  # argument types of the traced entry point
    return lib.attn_decode_global_traced(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(shape), FAKE, 1 << 30, FAKE,
                                         NULL)


def test_global_fp32_cache_is_valid_except_for_the_timeline(lib):
    # fp32 K=V caches run the fp32 kernel; the traced instance is bf16 only
    assert traced(lib, _gshape(kv_dtype=B.DA_DTYPE_F32)) == -2


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="needs a machine without a GPU")
def test_global_fp32_cache_reaches_the_device_check(lib):
    f32 = _gshape(kv_dtype=B.DA_DTYPE_F32)
    assert glob(lib, f32) == -4
    assert glob_noalloc(lib, f32) == -4
    assert global_gated(lib, f32) == -4
    assert traced(lib, _gshape()) == -4


def glob_noalloc(lib, shape, ptrs=None):
    p = ptrs or [FAKE] * 5
    return lib.attn_decode_global_noalloc(p[0], p[1], p[2], p[3], p[4], ctypes.byref(shape), NULL)


def test_global_noalloc_validation(lib):
    assert glob_noalloc(lib, _gshape(batch=-1)) == -1
    assert glob_noalloc(lib, _gshape(), ptrs=[FAKE, FAKE, FAKE, FAKE, NULL]) == -1
    assert glob_noalloc(lib, _gshape(group=8)) == -2
    assert glob_noalloc(lib, _gshape(batch=5000)) == -2
    assert glob_noalloc(lib, _gshape(batch=256, max_pages_per_seq=1 << 23)) == -2


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="needs a machine without a GPU")
def test_global_noalloc_no_device_after_valid_arguments(lib):
    assert glob_noalloc(lib, _gshape()) == -4


def test_workspace_bytes_with_explicit_splits(lib):
    assert da.attn_decode_global_workspace_bytes(_gshape(num_splits=1)) == 0
    n = da.attn_decode_global_workspace_bytes(_gshape(num_splits=10))
    assert n == 16384 + 2 * 10 * (16 * 512 + 32) * 4


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="needs a machine without a GPU")
def test_no_device_reported_after_valid_arguments(lib):
    assert sliding(lib, _shape()) == -4
    for ns in (1, 2, 4, 8):
        assert sliding(lib, _shape(num_splits=ns)) == -4
    assert glob(lib, _gshape()) == -4
    n = ctypes.c_size_t(0)
    assert lib.attn_decode_global_workspace_bytes(ctypes.byref(_gshape()), ctypes.byref(n)) == -4


def append_sliding(lib, shape, ptrs=None):
    p = ptrs or [FAKE] * 10
    return lib.attn_kv_append_sliding(*p, ctypes.byref(shape) if shape is not None else None, NULL)


def append_global(lib, shape, ptrs=None):
    p = ptrs or [FAKE] * 8
    return lib.attn_kv_append_global(*p, ctypes.byref(shape) if shape is not None else None, NULL)


def test_append_validation(lib):
    assert append_sliding(lib, None) == -1
    assert append_sliding(lib, _shape(batch=0)) == -1
    assert append_sliding(lib, _shape(), ptrs=[FAKE] * 9 + [NULL]) == -1
    assert append_sliding(lib, _shape(head_dim=512)) == -2
    assert append_global(lib, None) == -1
    assert append_global(lib, _gshape(), ptrs=[NULL] + [FAKE] * 7) == -1
    assert append_global(lib, _gshape(head_dim=256)) == -2
    s = _gshape()
    s.page_size = 8
    assert append_global(lib, s) == -2


def append_prenorm(lib, shape, ptrs=None):
    p = ptrs or [FAKE] * 7
    return lib.attn_kv_append_global_prenorm(*p, ctypes.byref(shape) if shape is not None else None, NULL)


def test_append_prenorm_validation(lib):
    assert append_prenorm(lib, None) == -1
    for i in range(7):  # every pointer argument is required
        ptrs = [FAKE] * 7
        ptrs[i] = NULL
        assert append_prenorm(lib, _gshape(), ptrs=ptrs) == -1
    assert append_prenorm(lib, _gshape(head_dim=256)) == -2
    s = _gshape()
    s.kv_dtype = B.DA_DTYPE_F32  # the pre-norm cache is bf16 only
    assert append_prenorm(lib, s) == -2


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="needs a machine without a GPU")
def test_append_no_device_reported_after_valid_arguments(lib):
    assert append_sliding(lib, _shape()) == -4
    assert append_global(lib, _gshape()) == -4
    assert append_prenorm(lib, _gshape()) == -4


def sliding_gated(lib, shape, gate=FAKE, ptrs=None):
    p = ptrs or [FAKE] * 6
    return lib.attn_decode_sliding_gated(p[0], p[1], p[2], p[3], p[4], 1024, gate, p[5],
                                         ctypes.byref(shape), NULL)


def global_gated(lib, shape, gate=FAKE, ptrs=None):
    p = ptrs or [FAKE] * 5
    return lib.attn_decode_global_gated(p[0], p[1], p[2], p[3], gate, p[4], ctypes.byref(shape),
                                        FAKE, 1 << 30, NULL)


def test_gated_validation(lib):
    assert sliding_gated(lib, _shape(), gate=NULL) == -1
    assert sliding_gated(lib, _shape(), ptrs=[FAKE] * 5 + [NULL]) == -1
    assert sliding_gated(lib, _shape(head_dim=512)) == -2
    assert global_gated(lib, _gshape(), gate=NULL) == -1
    assert global_gated(lib, _gshape(group=8)) == -2


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="needs a machine without a GPU")
def test_gated_no_device_reported_after_valid_arguments(lib):
    assert sliding_gated(lib, _shape()) == -4
    assert global_gated(lib, _gshape()) == -4


def mq(lib, shape, sliding=True, max_q=8, window=1024, ptrs=None):
    p = ptrs or [FAKE] * 7
    if sliding:
        return lib.attn_multiquery_sliding(p[0], p[1], max_q, p[2], p[3], p[4], p[5], window, p[6],
                                           ctypes.byref(shape), FAKE, 1 << 30, NULL)
    return lib.attn_multiquery_global(p[0], p[1], max_q, p[2], p[4], p[5], p[6], ctypes.byref(shape),
                                      FAKE, 1 << 30, NULL)


def test_multiquery_validation(lib):
    assert mq(lib, _shape(), max_q=0) == -1
    assert mq(lib, _shape(), window=-1) == -1
    assert mq(lib, _shape(), ptrs=[FAKE, NULL] + [FAKE] * 5) == -1
    assert mq(lib, _shape(kv_dtype=B.DA_DTYPE_F32)) == -2
    assert mq(lib, _shape(head_dim=512)) == -2
    assert mq(lib, _shape(), max_q=(1 << 18) + 1) == -2
    assert mq(lib, _gshape(), sliding=False, ptrs=[FAKE] * 6 + [NULL]) == -1
    assert mq(lib, _gshape(group=8), sliding=False) == -2
    n = ctypes.c_size_t(0)
    assert lib.attn_multiquery_workspace_bytes(ctypes.byref(_shape()), 0, 1024, ctypes.byref(n)) == -1
    assert lib.attn_multiquery_workspace_bytes(ctypes.byref(_shape()), 8, 1024, None) == -1


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="needs a machine without a GPU")
def test_multiquery_no_device_reported_after_valid_arguments(lib):
    assert mq(lib, _shape()) == -4
    assert mq(lib, _gshape(), sliding=False) == -4
    n = ctypes.c_size_t(0)
    assert lib.attn_multiquery_workspace_bytes(ctypes.byref(_gshape()), 8, 0, ctypes.byref(n)) == -4


def test_prenorm_validation(lib):
    def call(shape, ptrs=None, w=FAKE):
        p = ptrs or [FAKE] * 5
        return lib.attn_decode_global_prenorm(p[0], p[1], w, p[2], p[3], p[4], ctypes.byref(shape), FAKE, 1 << 30,
                                              NULL)
    assert call(_gshape(), w=NULL) == -1
    assert call(_gshape(), ptrs=[FAKE, NULL, FAKE, FAKE, FAKE]) == -1
    assert call(_gshape(group=8)) == -2
    assert call(_gshape(kv_dtype=B.DA_DTYPE_F32)) == -2


PROBE_HEADER = os.path.join(ROOT, "include", "decode_attn_probe.h")


def test_probe_library_exports_and_validates():
    from decode_attention_amd import probe as P
    if not os.path.exists(P.probe_library_path()):
        from decode_attention_amd.build import build
        build()
    plib = P.load_probe_library()
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"^\s*\w+\s+(da_probe_\w+)\s*\(", text, flags=re.M)))
    assert declared == sorted(P.EXPORTS)
    for name in declared:
        assert hasattr(plib, name), name
    f = plib.da_probe_read_pages
    assert f(NULL, FAKE, 4, 256, FAKE, NULL) == -1
    assert f(FAKE, NULL, 4, 256, FAKE, NULL) == -1
    assert f(FAKE, FAKE, 4, 256, NULL, NULL) == -1
    assert f(FAKE, FAKE, -1, 256, FAKE, NULL) == -1
    assert f(FAKE, FAKE, 4, 0, FAKE, NULL) == -1
    assert f(FAKE, FAKE, 4, 65536, FAKE, NULL) == -1
    assert f(ctypes.c_void_p(0x1008), FAKE, 4, 256, FAKE, NULL) == -1  # not 16-byte aligned
    assert f(FAKE, FAKE, 0, 256, FAKE, NULL) == 0  # nothing to read: nothing enqueued


def test_bind_records_and_replays_the_library_calls():
    # the mechanism alone, with a stand-in for a library function
    from decode_attention_amd import binding as B
    calls = []

    def cfunc(*args):
        calls.append(args)
        return 0

    def fn(x, y=0):
        B._call(cfunc, x, y)
        B._call(cfunc, y, x)
        return "result"

    run, result = B.bind(fn, 1, y=2)
    assert result == "result"
    assert calls == [(1, 2), (2, 1)]  # bind issues the recorded calls once
    run()
    run()
    assert calls == [(1, 2), (2, 1)] * 3
    with pytest.raises(B.DecodeAttnError):
        B.bind(lambda: None)  # nothing to bind

    def failing(*args):
        return -2
    run, _ = None, None
    with pytest.raises(B.DecodeAttnError):
        B.bind(lambda: B._call(failing))
    with pytest.raises(B.DecodeAttnError):
        B.bind(lambda: B.bind(fn, 1))  # no nesting
    assert getattr(B._capture, "rec", None) is None


def test_trace_summary_end_by_segments():
    # synthetic timeline entries: XCC 0 ends at 100 / 104 us (1 / 2
    # segments), XCC 1 at 110 / 114; relative to each XCC's mean the
    # one-segment workgroups sit 2 us early and the two-segment ones 2 late
    import numpy as np
    from decode_attention_amd import trace as T
    tick = 1.0 / T.TICK_US
    rows = []
    for xcc, base in ((0, 100.0), (1, 110.0)):
        for segs, extra in ((1, 0.0), (2, 4.0)):
            rows.append([1000, 1000 + round((base + extra) * tick), xcc | (segs << 8), 10])
    res = T.summarize(np.array(rows, dtype=np.int64))
    by = res["end_vs_xcc_mean_by_segments_us"]
    assert by[1][0] == 2 and by[2][0] == 2
    assert abs(by[1][1] + 2.0) < 1e-6 and abs(by[2][1] - 2.0) < 1e-6
    assert abs(res["per_xcc_end_mean_us"][0] - 102.0) < 1e-6
