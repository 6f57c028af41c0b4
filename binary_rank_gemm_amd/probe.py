"""Binding of the measurement probe (include/littlebit_probe.h): one
read-only streaming pass over a device buffer, the reference the benchmark
reads its decode bandwidth against.  Not part of the method."""
from __future__ import annotations

import ctypes as C

from ._binding import _check, _stream, lib

EXPORTS = ["lb_probe_stream_read"]


def _fn():
    f = lib().lb_probe_stream_read
    f.restype = C.c_int
    f.argtypes = [C.c_void_p, C.c_int64, C.c_void_p]
    return f


def stream_read(buf, stream=None) -> None:
    """Enqueue lb_probe_stream_read over a contiguous device tensor."""
    _check(_fn()(C.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(), _stream(stream)))
