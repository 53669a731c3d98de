"""ctypes binding of ``libdecode_attn_probe.so`` (include/decode_attn_probe.h):
an HBM read probe with the decode kernels' page access pattern, used to put
their bandwidth next to what that pattern reaches on the device. Not part
of the attention path."""

import ctypes
import os
import threading

from .binding import DecodeAttnError, _check, _stream

HERE = os.path.dirname(os.path.abspath(__file__))
PAGE_BYTES = 16384
EXPORTS = ("da_probe_read_pages",)

_lock = threading.Lock()
_lib = None


def probe_library_path():
    return os.path.join(HERE, "lib", "libdecode_attn_probe.so")


def load_probe_library():
    """Load the probe library (raises DecodeAttnError if it is not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = probe_library_path()
        if not os.path.exists(path):
            raise DecodeAttnError(-100, f"probe library not built: {path} "
                                        "(run `python -m decode_attention_amd.build`)")
        lib = ctypes.CDLL(path)
        lib.da_probe_read_pages.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p]
        lib.da_probe_read_pages.restype = ctypes.c_int32
        _lib = lib
        return lib


def read_pages(buf, page_ids, workgroups, sink, stream=None, check_ids=True):
    """Reads the 16 KB pages of `buf` (a cuda tensor) that `page_ids` (cuda
    int32) lists, in that order, on the current stream. check_ids=False
    skips the range check of the ids (a device reduction and a host sync per
    call): for timing loops over ids already checked once."""
    import torch
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous cuda tensor")
    if not (page_ids.is_cuda and page_ids.dtype == torch.int32 and page_ids.is_contiguous()
            and page_ids.device == buf.device):
        raise ValueError("page_ids must be contiguous cuda int32 on buf's device")
    if not (sink.is_cuda and sink.numel() >= 1 and sink.element_size() == 4):
        raise ValueError("sink must be a cuda tensor of at least one 4-byte element")
    n_pages = buf.numel() * buf.element_size() // PAGE_BYTES
    if page_ids.numel() == 0:
        return  # nothing to read (an empty tensor has no device address to pass)
    if check_ids:
        lo, hi = int(page_ids.min()), int(page_ids.max())
        if lo < 0 or hi >= n_pages:
            raise ValueError(f"page ids must lie in [0, {n_pages})")
    _check(load_probe_library().da_probe_read_pages(
        ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(page_ids.data_ptr()), int(page_ids.numel()),
        int(workgroups), ctypes.c_void_p(sink.data_ptr()), _stream(stream)))
