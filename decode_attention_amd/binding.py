"""ctypes binding of ``libdecode_attn.so`` (declared in include/decode_attn.h).

Argument marshalling only: shape and dtype checks on torch tensors, the
``da_shape`` struct, output/workspace allocation through torch, and the
current torch stream. Every step of the computation runs in the library's HIP
kernels; there is no fallback path. If the library is missing the calls raise.
"""

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))

DA_OK = 0
DA_DTYPE_F32 = 0
DA_DTYPE_BF16 = 1
PAGE_SIZE = 16

_lock = threading.Lock()
_lib = None
_workspaces = {}


class DecodeAttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class DaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
    ]


EXPORTS = ("attn_decode_sliding", "attn_decode_global", "attn_decode_global_workspace_bytes",
           "attn_decode_global_noalloc",
           "attn_decode_sliding_gated", "attn_decode_global_gated", "attn_decode_global_prenorm",
           "attn_kv_append_sliding", "attn_kv_append_global", "attn_kv_append_global_prenorm",
           "attn_multiquery_sliding", "attn_multiquery_global", "attn_multiquery_workspace_bytes",
           "attn_status_string")


def library_path():
    return os.environ.get("DECODE_ATTN_LIB", os.path.join(HERE, "lib", "libdecode_attn.so"))


def load_library():
    """Load the shared library (raises DecodeAttnError if it is not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise DecodeAttnError(-100, f"HIP library not built: {path} "
                                        "(run `python -m decode_attention_amd.build`)")
        lib = ctypes.CDLL(path)
        vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
        lib.attn_decode_sliding.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int32, vp,
                                            ctypes.POINTER(DaShape), vp]
        lib.attn_decode_sliding.restype = ctypes.c_int32
        lib.attn_decode_global.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(DaShape), vp,
                                           ctypes.c_size_t, vp]
        lib.attn_decode_global.restype = ctypes.c_int32
        lib.attn_decode_global_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(DaShape), vp]
        lib.attn_decode_global_noalloc.restype = ctypes.c_int32
        lib.attn_decode_sliding_gated.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp,
                                                  ctypes.POINTER(DaShape), vp]
        lib.attn_decode_sliding_gated.restype = ctypes.c_int32
        lib.attn_decode_global_gated.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(DaShape), vp,
                                                 ctypes.c_size_t, vp]
        lib.attn_decode_global_gated.restype = ctypes.c_int32
        lib.attn_decode_global_prenorm.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(DaShape), vp,
                                                   ctypes.c_size_t, vp]
        lib.attn_decode_global_prenorm.restype = ctypes.c_int32
        lib.attn_decode_global_workspace_bytes.argtypes = [ctypes.POINTER(DaShape),
                                                           ctypes.POINTER(ctypes.c_size_t)]
        lib.attn_decode_global_workspace_bytes.restype = ctypes.c_int32
        lib.attn_kv_append_sliding.argtypes = [vp] * 10 + [ctypes.POINTER(DaShape), vp]
        lib.attn_kv_append_sliding.restype = ctypes.c_int32
        lib.attn_kv_append_global.argtypes = [vp] * 8 + [ctypes.POINTER(DaShape), vp]
        lib.attn_kv_append_global.restype = ctypes.c_int32
        lib.attn_kv_append_global_prenorm.argtypes = [vp] * 7 + [ctypes.POINTER(DaShape), vp]
        lib.attn_kv_append_global_prenorm.restype = ctypes.c_int32
        lib.attn_multiquery_sliding.argtypes = [vp, vp, ctypes.c_int32, vp, vp, vp, vp, ctypes.c_int32, vp,
                                                ctypes.POINTER(DaShape), vp, ctypes.c_size_t, vp]
        lib.attn_multiquery_sliding.restype = ctypes.c_int32
        lib.attn_multiquery_global.argtypes = [vp, vp, ctypes.c_int32, vp, vp, vp, vp, ctypes.POINTER(DaShape), vp,
                                               ctypes.c_size_t, vp]
        lib.attn_multiquery_global.restype = ctypes.c_int32
        lib.attn_multiquery_workspace_bytes.argtypes = [ctypes.POINTER(DaShape), ctypes.c_int32, ctypes.c_int32,
                                                        ctypes.POINTER(ctypes.c_size_t)]
        lib.attn_multiquery_workspace_bytes.restype = ctypes.c_int32
        lib.attn_status_string.argtypes = [ctypes.c_int32]
        lib.attn_status_string.restype = ctypes.c_char_p
        del i32p
        _lib = lib
        return lib


def attn_status_string(status):
    return load_library().attn_status_string(int(status)).decode()


def _check(status):
    if status != DA_OK:
        raise DecodeAttnError(status, attn_status_string(status))


_capture = threading.local()


def _call(cfunc, *args):
    """Issues one library call (a kernel launch), or records it while bind()
    prepares a bound call."""
    rec = getattr(_capture, "rec", None)
    if rec is not None:
        rec.append((cfunc, args))
        return
    _check(cfunc(*args))


def bind(fn, *args, **kwargs):
    """Prepares a call for a loop that repeats it on the same tensors.

    Runs fn(*args, **kwargs), one of this module's calls, with its argument
    checks and conversions, records the library call(s) it makes instead of
    issuing them, and returns (run, result). result is what fn returns (keep
    it, and every tensor passed, alive while run is used). run() issues the
    same library call(s) again, with the same device pointers, shape and
    stream, skipping the Python-side checks. The library still validates
    its arguments on each call. The caller must not resize, free or
    reallocate the tensors, and should use the stream that was current at
    bind time, or the one passed. run is issued once before bind returns.
    """
    if getattr(_capture, "rec", None) is not None:
        raise DecodeAttnError(-1, "bind() calls do not nest")
    _capture.rec = []
    try:
        result = fn(*args, **kwargs)
        rec = _capture.rec
    finally:
        _capture.rec = None
    if not rec:
        raise DecodeAttnError(-1, "the call issued no library call to bind")

    def run():
        for cfunc, a in rec:
            st = cfunc(*a)
            if st != DA_OK:
                raise DecodeAttnError(st, attn_status_string(st))

    run()
    return run, result


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return DA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DA_DTYPE_BF16
    raise DecodeAttnError(-1, f"unsupported tensor dtype {t.dtype}")


def _require(cond, msg):
    if not cond:
        raise DecodeAttnError(-1, msg)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_shape(batch, num_kv_heads, group, head_dim, max_pages_per_seq, num_pages, kv_dtype,
               num_splits=0, out_dtype=DA_DTYPE_F32):
    return DaShape(int(batch), int(num_kv_heads), int(group), int(head_dim), PAGE_SIZE,
                   int(max_pages_per_seq), int(num_pages), int(kv_dtype), int(out_dtype),
                   int(num_splits))


def _decode_out(out, shape, device):
    """The decode calls' output: allocated fp32 when not given, else a
    contiguous fp32 or bf16 tensor of that shape; returns (out, dtype code)."""
    import torch
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=device)
    _require(out.dtype in (torch.float32, torch.bfloat16) and out.is_contiguous() and tuple(out.shape) == shape
             and out.device == device, f"out must be contiguous fp32 or bf16 {list(shape)} on q's device")
    return out, (DA_DTYPE_BF16 if out.dtype == torch.bfloat16 else DA_DTYPE_F32)


def _check_common(q, block_table, seq_lens, caches):
    import torch
    _require(q.is_cuda and q.dim() == 3 and q.is_contiguous(), "q must be a contiguous cuda [B, Hq, D] tensor")
    for c in caches:
        _require(c.is_cuda and c.is_contiguous() and c.device == q.device, "caches must be contiguous, on q's device")
        _require(c.dtype == q.dtype, "caches must have q's dtype")
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous()
             and block_table.device == q.device, "block_table must be contiguous int32 [B, P_max] on q's device")
    _require(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1 and seq_lens.is_contiguous()
             and seq_lens.device == q.device, "seq_lens must be contiguous int32 [B] on q's device")
    _require(block_table.shape[0] == q.shape[0] and seq_lens.shape[0] == q.shape[0], "batch mismatch")


def _check_gate(gate, out):
    import torch
    _require(gate.dtype == torch.float32 and gate.is_contiguous() and gate.device == out.device
             and gate.shape == out.shape, "gate must be contiguous fp32 with out's shape, on out's device")
    g0, o0 = gate.data_ptr(), out.data_ptr()
    n = out.numel() * 4
    _require(g0 + n <= o0 or o0 + n <= g0, "gate must not overlap out")


def attn_decode_sliding(q, k_cache, v_cache, block_table, seq_lens, window, out=None, stream=None, num_splits=0):
    """slidingDecodeGQA. q [B, Hkv*G, D]; k_cache, v_cache [P, Hkv, 16, D]
    (row-major pages); block_table int32 [B, P_max]; seq_lens int32 [B].
    Returns out [B, Hkv*G, D]: fp32 (allocated if not given) or the given
    fp32 or bf16 tensor. num_splits: waves each (sequence, KV head) window is
    divided among (0: the default, 4; or 1, 2, 4, 8)."""
    return _sliding(q, k_cache, v_cache, block_table, seq_lens, window, None, out, stream, num_splits)


def attn_decode_sliding_gated(q, k_cache, v_cache, block_table, seq_lens, window, gate, out=None, stream=None,
                              num_splits=0):
    """attn_decode_sliding followed by sigmoidGate: out = o * sigmoid(gate),
    gate fp32 [B, Hkv*G, D]."""
    return _sliding(q, k_cache, v_cache, block_table, seq_lens, window, gate, out, stream, num_splits)


def _sliding(q, k_cache, v_cache, block_table, seq_lens, window, gate, out, stream, num_splits=0):
    import torch
    lib = load_library()
    _check_common(q, block_table, seq_lens, (k_cache, v_cache))
    _require(k_cache.dim() == 4 and k_cache.shape == v_cache.shape and k_cache.shape[2] == PAGE_SIZE,
             "k_cache/v_cache must be [P, Hkv, 16, D]")
    B, Hq, D = q.shape
    P, Hkv, _, Dk = k_cache.shape
    _require(Dk == D and Hq % Hkv == 0, "head shape mismatch")
    out, out_dtype = _decode_out(out, (B, Hq, D), q.device)
    shape = make_shape(B, Hkv, Hq // Hkv, D, block_table.shape[1], P, _dtype_code(q), num_splits=num_splits,
                       out_dtype=out_dtype)
    if gate is None:
        _call(lib.attn_decode_sliding, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
              _ptr(seq_lens), int(window), _ptr(out), ctypes.byref(shape),
              _stream(stream))
    else:
        _check_gate(gate, out)
        _call(lib.attn_decode_sliding_gated, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
              _ptr(seq_lens), int(window), _ptr(gate), _ptr(out),
              ctypes.byref(shape), _stream(stream))
    return out


def _global_shape(q, kv_cache, block_table, num_splits, out_dtype=DA_DTYPE_F32):
    B, Hq, D = q.shape
    _require(kv_cache.dim() == 5 and kv_cache.shape[3] == PAGE_SIZE,
             "kv_cache must be tiled [P, Hkv, D/x, 16, x]")
    P, Hkv, nx, _, x = kv_cache.shape
    _require(nx * x == D and Hq % Hkv == 0, "head shape mismatch")
    return make_shape(B, Hkv, Hq // Hkv, D, block_table.shape[1], P, _dtype_code(q), num_splits, out_dtype)


def attn_decode_global_workspace_bytes(shape):
    n = ctypes.c_size_t(0)
    _check(load_library().attn_decode_global_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)))
    return int(n.value)


def attn_decode_global(q, kv_cache, block_table, seq_lens, out=None, workspace=None, num_splits=0,
                       stream=None):
    """decodeGQA with values = keys. q [B, Hkv*G, D]; kv_cache tiled
    [P, Hkv, D/x, 16, x]; returns out [B, Hkv*G, D] (fp32 if allocated here,
    else the given fp32 or bf16 tensor). When no workspace is
    given, one is allocated and cached per device, stream and size (calls on
    one stream run in order, so they may share it)."""
    return _global(q, kv_cache, block_table, seq_lens, None, out, workspace, num_splits, stream)


def attn_decode_global_noalloc(q, kv_cache, block_table, seq_lens, out, num_splits=0, stream=None):
    """attn_decode_global on the library's own device scratch array: the
    library call allocates nothing, and neither does this wrapper (out is
    required). Calls that may overlap on one device race."""
    import torch
    lib = load_library()
    _check_common(q, block_table, seq_lens, (kv_cache,))
    _require(out is not None, "out is required")
    out, out_dtype = _decode_out(out, tuple(q.shape), q.device)
    shape = _global_shape(q, kv_cache, block_table, num_splits, out_dtype)
    _call(lib.attn_decode_global_noalloc, _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
          _ptr(out), ctypes.byref(shape), _stream(stream))
    return out


def attn_decode_global_gated(q, kv_cache, block_table, seq_lens, gate, out=None, workspace=None, num_splits=0,
                             stream=None):
    """attn_decode_global followed by sigmoidGate: out = o * sigmoid(gate),
    gate fp32 [B, Hkv*G, D]."""
    return _global(q, kv_cache, block_table, seq_lens, gate, out, workspace, num_splits, stream)


def attn_decode_global_prenorm(q, x_cache, w_k, block_table, seq_lens, out=None, workspace=None, num_splits=0,
                               stream=None):
    """decodeGQA over the pre-norm cache: k = rope(rmsnorm(x, w_k)), v =
    rmsnormUnit(x) derived in the kernel. q bf16 [B, 16, 512]; x_cache bf16
    [P, 1, 64, 16, 8] (pre-norm layout); w_k fp32 [512]."""
    import torch
    _require(w_k.dtype == torch.float32 and w_k.is_contiguous() and w_k.device == q.device
             and tuple(w_k.shape) == (512,), "w_k must be contiguous fp32 [512] on q's device")
    return _global(q, x_cache, block_table, seq_lens, None, out, workspace, num_splits, stream, w_k=w_k)


def _global(q, kv_cache, block_table, seq_lens, gate, out, workspace, num_splits, stream, w_k=None):
    import torch
    lib = load_library()
    _check_common(q, block_table, seq_lens, (kv_cache,))
    out, out_dtype = _decode_out(out, tuple(q.shape), q.device)
    shape = _global_shape(q, kv_cache, block_table, num_splits, out_dtype)
    need = attn_decode_global_workspace_bytes(shape)
    st = _stream(stream)
    if workspace is None and need > 0:
        key = (q.device, st.value, need)
        workspace = _workspaces.get(key)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            _workspaces[key] = workspace
    ws_ptr = _ptr(workspace) if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if w_k is not None:
        _call(lib.attn_decode_global_prenorm, _ptr(q), _ptr(kv_cache), _ptr(w_k), _ptr(block_table),
              _ptr(seq_lens), _ptr(out), ctypes.byref(shape), ws_ptr, ws_bytes, st)
    elif gate is None:
        _call(lib.attn_decode_global, _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), _ptr(out),
              ctypes.byref(shape), ws_ptr, ws_bytes, st)
    else:
        _check_gate(gate, out)
        _call(lib.attn_decode_global_gated, _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
              _ptr(gate), _ptr(out), ctypes.byref(shape), ws_ptr, ws_bytes, st)
    return out


def _check_f32(name, t, shape, device):
    import torch
    _require(t.dtype == torch.float32 and t.is_contiguous() and t.device == device and tuple(t.shape) == shape,
             f"{name} must be contiguous fp32 {list(shape)} on the caches' device")


def attn_kv_append_sliding(q_raw, k_raw, v_raw, w_q, w_k, block_table, positions, k_cache, v_cache,
                           q_out=None, stream=None):
    """Norm + RoPE of the new tokens of a sliding layer and their append:
    q_raw fp32 [B, Hq, 256], k_raw/v_raw fp32 [B, Hkv, 256], w_q/w_k fp32
    [256], positions int32 [B]; writes k/v into their slots of k_cache/v_cache
    [P, Hkv, 16, 256] and returns q_out [B, Hq, 256] in the caches' dtype."""
    import torch
    lib = load_library()
    _require(k_cache.dim() == 4 and k_cache.shape == v_cache.shape and k_cache.shape[2] == PAGE_SIZE
             and k_cache.is_contiguous() and v_cache.is_contiguous() and k_cache.dtype == v_cache.dtype
             and k_cache.is_cuda and v_cache.device == k_cache.device,
             "k_cache/v_cache must be contiguous [P, Hkv, 16, D] on one device")
    P, Hkv, _, D = k_cache.shape
    B, Hq = q_raw.shape[0], q_raw.shape[1]
    dev = k_cache.device
    _check_f32("q_raw", q_raw, (B, Hq, D), dev)
    _check_f32("k_raw", k_raw, (B, Hkv, D), dev)
    _check_f32("v_raw", v_raw, (B, Hkv, D), dev)
    _check_f32("w_q", w_q, (D,), dev)
    _check_f32("w_k", w_k, (D,), dev)
    _require(Hq % Hkv == 0, "head shape mismatch")
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous()
             and block_table.shape[0] == B and block_table.device == dev, "block_table must be int32 [B, P_max]")
    _require(positions.dtype == torch.int32 and tuple(positions.shape) == (B,) and positions.is_contiguous()
             and positions.device == dev, "positions must be int32 [B]")
    if q_out is None:
        q_out = torch.empty((B, Hq, D), dtype=k_cache.dtype, device=dev)
    _require(q_out.dtype == k_cache.dtype and q_out.is_contiguous() and tuple(q_out.shape) == (B, Hq, D),
             "q_out must be contiguous [B, Hq, D] in the caches' dtype")
    shape = make_shape(B, Hkv, Hq // Hkv, D, block_table.shape[1], P, _dtype_code(k_cache))
    _call(lib.attn_kv_append_sliding, _ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(w_q), _ptr(w_k),
          _ptr(block_table), _ptr(positions), _ptr(k_cache), _ptr(v_cache),
          _ptr(q_out), ctypes.byref(shape), _stream(stream))
    return q_out


def attn_kv_append_global(q_raw, kv_raw, w_q, w_k, block_table, positions, kv_cache, q_out=None, stream=None):
    """Norm + RoPE of the new tokens of a global layer and the append of k to
    the tiled K=V cache [P, Hkv, D/x, 16, x]: q_raw fp32 [B, Hq, 512], kv_raw
    fp32 [B, Hkv, 512], w_q/w_k fp32 [512], positions int32 [B]; returns q_out
    [B, Hq, 512] in the cache's dtype."""
    import torch
    lib = load_library()
    _require(kv_cache.dim() == 5 and kv_cache.shape[3] == PAGE_SIZE and kv_cache.is_contiguous()
             and kv_cache.is_cuda, "kv_cache must be contiguous tiled [P, Hkv, D/x, 16, x]")
    P, Hkv, nx, _, x = kv_cache.shape
    D = nx * x
    B, Hq = q_raw.shape[0], q_raw.shape[1]
    dev = kv_cache.device
    _check_f32("q_raw", q_raw, (B, Hq, D), dev)
    _check_f32("kv_raw", kv_raw, (B, Hkv, D), dev)
    _check_f32("w_q", w_q, (D,), dev)
    _check_f32("w_k", w_k, (D,), dev)
    _require(Hq % Hkv == 0 and x * kv_cache.element_size() == 16, "head shape mismatch")
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous()
             and block_table.shape[0] == B and block_table.device == dev, "block_table must be int32 [B, P_max]")
    _require(positions.dtype == torch.int32 and tuple(positions.shape) == (B,) and positions.is_contiguous()
             and positions.device == dev, "positions must be int32 [B]")
    if q_out is None:
        q_out = torch.empty((B, Hq, D), dtype=kv_cache.dtype, device=dev)
    _require(q_out.dtype == kv_cache.dtype and q_out.is_contiguous() and tuple(q_out.shape) == (B, Hq, D),
             "q_out must be contiguous [B, Hq, D] in the cache's dtype")
    shape = make_shape(B, Hkv, Hq // Hkv, D, block_table.shape[1], P, _dtype_code(kv_cache))
    _call(lib.attn_kv_append_global, _ptr(q_raw), _ptr(kv_raw), _ptr(w_q), _ptr(w_k), _ptr(block_table),
          _ptr(positions), _ptr(kv_cache), _ptr(q_out), ctypes.byref(shape),
          _stream(stream))
    return q_out


def attn_kv_append_global_prenorm(q_raw, x_raw, w_q, block_table, positions, x_cache, q_out=None, stream=None):
    """Norm + RoPE of the new tokens' q of a global layer, and the append of
    their shared projection x, unnormalised, to the bf16 pre-norm cache
    [P, Hkv, 64, 16, 8] that attn_decode_global_prenorm reads: q_raw fp32
    [B, Hq, 512], x_raw fp32 [B, Hkv, 512], w_q fp32 [512], positions int32
    [B]; returns q_out bf16 [B, Hq, 512]."""
    import torch
    lib = load_library()
    _require(x_cache.dim() == 5 and x_cache.dtype == torch.bfloat16 and tuple(x_cache.shape[2:]) == (64, PAGE_SIZE, 8)
             and x_cache.is_contiguous() and x_cache.is_cuda, "x_cache must be contiguous bf16 [P, Hkv, 64, 16, 8]")
    P, Hkv = x_cache.shape[0], x_cache.shape[1]
    D = 512
    B, Hq = q_raw.shape[0], q_raw.shape[1]
    dev = x_cache.device
    _check_f32("q_raw", q_raw, (B, Hq, D), dev)
    _check_f32("x_raw", x_raw, (B, Hkv, D), dev)
    _check_f32("w_q", w_q, (D,), dev)
    _require(Hq % Hkv == 0, "head shape mismatch")
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous()
             and block_table.shape[0] == B and block_table.device == dev, "block_table must be int32 [B, P_max]")
    _require(positions.dtype == torch.int32 and tuple(positions.shape) == (B,) and positions.is_contiguous()
             and positions.device == dev, "positions must be int32 [B]")
    if q_out is None:
        q_out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    _require(q_out.dtype == torch.bfloat16 and q_out.is_contiguous() and tuple(q_out.shape) == (B, Hq, D),
             "q_out must be contiguous bf16 [B, Hq, D]")
    shape = make_shape(B, Hkv, Hq // Hkv, D, block_table.shape[1], P, DA_DTYPE_BF16)
    _call(lib.attn_kv_append_global_prenorm, _ptr(q_raw), _ptr(x_raw), _ptr(w_q), _ptr(block_table),
          _ptr(positions), _ptr(x_cache), _ptr(q_out), ctypes.byref(shape),
          _stream(stream))
    return q_out


def attn_multiquery_workspace_bytes(shape, max_queries, window=0):
    n = ctypes.c_size_t(0)
    _check(load_library().attn_multiquery_workspace_bytes(ctypes.byref(shape), int(max_queries), int(window),
                                                          ctypes.byref(n)))
    return int(n.value)


def _workspace(device, st, need):
    import torch
    key = (device, st.value, need)
    ws = _workspaces.get(key)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _multiquery(sliding, q, q_start, max_queries, caches, block_table, seq_lens, window, out, workspace,
                num_splits, stream):
    import torch
    lib = load_library()
    _require(q.is_cuda and q.dim() == 3 and q.is_contiguous() and q.dtype == torch.bfloat16,
             "q must be a contiguous bf16 cuda [T, Hq, D] tensor")
    for c in caches:
        _require(c.is_cuda and c.is_contiguous() and c.device == q.device and c.dtype == q.dtype,
                 "caches must be contiguous bf16, on q's device")
    B = seq_lens.shape[0]
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous()
             and block_table.device == q.device and block_table.shape[0] == B,
             "block_table must be contiguous int32 [B, P_max] on q's device")
    _require(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1 and seq_lens.is_contiguous()
             and seq_lens.device == q.device, "seq_lens must be contiguous int32 [B] on q's device")
    _require(q_start.dtype == torch.int32 and q_start.dim() == 1 and q_start.is_contiguous()
             and q_start.device == q.device and q_start.shape[0] == B + 1,
             "q_start must be contiguous int32 [B + 1] on q's device")
    T, Hq, D = q.shape
    if sliding:
        k_cache = caches[0]
        _require(k_cache.dim() == 4 and k_cache.shape == caches[1].shape and k_cache.shape[2] == PAGE_SIZE,
                 "k_cache/v_cache must be [P, Hkv, 16, D]")
        P, Hkv, _, Dk = k_cache.shape
        _require(Dk == D and Hq % Hkv == 0, "head shape mismatch")
    else:
        kv = caches[0]
        _require(kv.dim() == 5 and kv.shape[3] == PAGE_SIZE, "kv_cache must be tiled [P, Hkv, D/x, 16, x]")
        P, Hkv, nx, _, x = kv.shape
        _require(nx * x == D and Hq % Hkv == 0, "head shape mismatch")
    shape = make_shape(B, Hkv, Hq // Hkv, D, block_table.shape[1], P, _dtype_code(q), num_splits)
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    _require(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (T, Hq, D),
             "out must be contiguous fp32 [T, Hq, D]")
    if T == 0:
        return out  # no query rows: nothing to compute (the C call needs non-NULL q and out)
    st = _stream(stream)
    need = attn_multiquery_workspace_bytes(shape, max_queries, window)
    if workspace is None and need > 0:
        workspace = _workspace(q.device, st, need)
    ws_ptr = _ptr(workspace) if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if sliding:
        _call(lib.attn_multiquery_sliding, _ptr(q), _ptr(q_start), int(max_queries), _ptr(caches[0]),
              _ptr(caches[1]), _ptr(block_table), _ptr(seq_lens), int(window),
              _ptr(out), ctypes.byref(shape), ws_ptr, ws_bytes, st)
    else:
        _call(lib.attn_multiquery_global, _ptr(q), _ptr(q_start), int(max_queries), _ptr(caches[0]),
              _ptr(block_table), _ptr(seq_lens), _ptr(out), ctypes.byref(shape),
              ws_ptr, ws_bytes, st)
    return out


def attn_multiquery_sliding(q, q_start, max_queries, k_cache, v_cache, block_table, seq_lens, window, out=None,
                            workspace=None, num_splits=0, stream=None):
    """slidingGQA for several queries per sequence at its last positions:
    q bf16 [T, Hq, 256] (sequence b's rows q_start[b]..q_start[b+1]-1,
    query s at position L - S_b + s); k_cache, v_cache [P, Hkv, 16, 256];
    returns out fp32 [T, Hq, 256]. max_queries >= every S_b."""
    return _multiquery(True, q, q_start, max_queries, (k_cache, v_cache), block_table, seq_lens, window, out,
                       workspace, num_splits, stream)


def attn_multiquery_global(q, q_start, max_queries, kv_cache, block_table, seq_lens, out=None, workspace=None,
                           num_splits=0, stream=None):
    """causalGQA for several queries per sequence at its last positions, with
    values = keys: q bf16 [T, 16, 512], kv_cache tiled [P, 1, 64, 16, 8];
    returns out fp32 [T, 16, 512]."""
    return _multiquery(False, q, q_start, max_queries, (kv_cache,), block_table, seq_lens, 0, out, workspace,
                       num_splits, stream)
