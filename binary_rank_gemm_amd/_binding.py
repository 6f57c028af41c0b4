"""ctypes binding of liblittlebit (argument marshalling only).

Every step of the forward runs in the library's HIP kernels; torch is used
here only to own device memory and to name the current HIP stream.  The
library must have been built (``binary_rank_gemm_amd.build.build()``): if it
is missing, loading raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# LITTLEBIT_LIB names another build of the library (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("LITTLEBIT_LIB") or os.path.join(HERE, "liblittlebit.so")

OK, INVALID_ARGUMENT, INVALID_SIGN, ALIGNMENT, UNSUPPORTED, OUT_OF_MEMORY, HIP_ERROR = range(7)
BF16, FP32, BF16_FP32 = 0, 1, 2   # lb_dtype: element types of (x, y)
REGIME_AUTO, REGIME_EXACT, REGIME_DECODE, REGIME_PREFILL = 0, 1, 2, 3

STATUS_NAMES = {OK: "LB_OK", INVALID_ARGUMENT: "LB_ERR_INVALID_ARGUMENT", INVALID_SIGN: "LB_ERR_INVALID_SIGN",
                ALIGNMENT: "LB_ERR_ALIGNMENT", UNSUPPORTED: "LB_ERR_UNSUPPORTED",
                OUT_OF_MEMORY: "LB_ERR_OUT_OF_MEMORY", HIP_ERROR: "LB_ERR_HIP"}

# every symbol include/littlebit.h declares (the measurement probe of
# include/littlebit_probe.h is bound in probe.py)
EXPORTS = [
    "lb_packed_words_per_row", "lb_rank_for_bpw", "lb_pack_signs_host", "lb_pack_signs", "lb_unpack_signs",
    "lb_linear_create", "lb_linear_forward", "lb_linear_forward_ex", "lb_linear_forward_noalloc", "lb_auto_regime",
    "lb_linear_info",
    "lb_linear_destroy",
    "lb_stack_create", "lb_stack_forward", "lb_stack_forward_ex", "lb_stack_set_persistent",
    "lb_stack_persistent_status", "lb_stack_destroy", "lb_status_string",
    "lb_last_error", "lb_init_dual_svid",
]


class LbPath(C.Structure):
    _fields_ = [("rank", C.c_int64), ("u_packed", C.c_void_p), ("v_packed", C.c_void_p),
                ("h", C.c_void_p), ("g", C.c_void_p), ("l", C.c_void_p)]


class LbPathInit(C.Structure):
    _fields_ = [("rank", C.c_int64), ("u_packed", C.c_void_p), ("v_packed", C.c_void_p),
                ("h", C.c_void_p), ("g", C.c_void_p), ("l", C.c_void_p)]


class LittleBitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with binary_rank_gemm_amd.build.build()")
    L = C.CDLL(LIB_PATH)
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
    sig = {
        "lb_packed_words_per_row": (i64, [i64]),
        "lb_rank_for_bpw": (i64, [i64, i64, i64, i64]),
        "lb_pack_signs_host": (C.c_int, [vp, i64, i64, vp]),
        "lb_pack_signs": (C.c_int, [vp, i64, i64, vp, vp]),
        "lb_unpack_signs": (C.c_int, [vp, i64, i64, vp, vp]),
        "lb_linear_create": (C.c_int, [i64, i64, C.POINTER(LbPath), i32, vp, C.POINTER(vp)]),
        "lb_linear_forward": (C.c_int, [vp, vp, vp, i64, C.c_int, vp]),
        "lb_linear_forward_ex": (C.c_int, [vp, vp, vp, i64, C.c_int, C.c_int, vp]),
        "lb_linear_forward_noalloc": (C.c_int, [vp, vp, vp, i64, C.c_int, vp]),
        "lb_auto_regime": (C.c_int, [C.POINTER(vp), i32, i64, C.c_int, C.POINTER(C.c_int)]),
        "lb_linear_info": (C.c_int, [vp, C.POINTER(i64), C.POINTER(i64), C.POINTER(i32), C.POINTER(i64),
                                     C.POINTER(i64)]),
        "lb_linear_destroy": (C.c_int, [vp]),
        "lb_stack_create": (C.c_int, [C.POINTER(vp), i32, C.POINTER(vp)]),
        "lb_stack_forward": (C.c_int, [vp, C.POINTER(vp), C.POINTER(vp), i64, C.c_int, vp]),
        "lb_stack_forward_ex": (C.c_int, [vp, C.POINTER(vp), C.POINTER(vp), i64, C.c_int, C.c_int, i32, vp]),
        "lb_stack_set_persistent": (C.c_int, [vp, i32]),
        "lb_stack_persistent_status": (C.c_int, [vp, C.POINTER(i32), C.POINTER(i32)]),
        "lb_stack_destroy": (C.c_int, [vp]),
        "lb_status_string": (C.c_char_p, [C.c_int]),
        "lb_last_error": (C.c_char_p, []),
        "lb_init_dual_svid": (C.c_int, [vp, i64, i64, vp, i32, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != OK:
        raise LittleBitError(status, lib().lb_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def packed_words_per_row(rank: int) -> int:
    return int(lib().lb_packed_words_per_row(rank))


def rank_for_bpw(d_out: int, d_in: int, bpw_num: int, bpw_den: int) -> int:
    return int(lib().lb_rank_for_bpw(d_out, d_in, bpw_num, bpw_den))


def pack_signs_host(signs: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(signs, dtype=np.int8)
    if s.ndim != 2:
        raise ValueError("signs must be [rows, rank]")
    rows, rank = s.shape
    out = np.zeros((rows, packed_words_per_row(rank)), dtype=np.uint32)
    _check(lib().lb_pack_signs_host(s.ctypes.data, rows, rank, out.ctypes.data))
    return out


def pack_signs(signs, stream=None):
    """Device int8 [rows, rank] tensor -> device int32 [rows, ceil(rank/32)] tensor."""
    import torch
    rows, rank = signs.shape
    out = torch.zeros((rows, packed_words_per_row(rank)), dtype=torch.int32, device=signs.device)
    _check(lib().lb_pack_signs(signs.data_ptr(), rows, rank, out.data_ptr(), _stream(stream)))
    return out


def unpack_signs(packed, rank: int, stream=None):
    import torch
    rows = packed.shape[0]
    out = torch.empty((rows, rank), dtype=torch.int8, device=packed.device)
    _check(lib().lb_unpack_signs(packed.data_ptr(), rows, rank, out.data_ptr(), _stream(stream)))
    return out


def init_dual_svid(W, ranks: Sequence[int], stream=None) -> List[Dict]:
    """Dual-SVID initialisation of a layer from a dense fp32 device tensor W
    [d_out, d_in] (lb_init_dual_svid): one dict per path of device tensors u
    (int32 [d_out, words]), v (int32 [d_in, words]), h, g, l (int16 fp16 bits),
    ready for Linear(d_out, d_in, paths)."""
    import torch
    if W.dim() != 2 or W.dtype != torch.float32 or not W.is_contiguous():
        raise ValueError("W must be a contiguous float32 [d_out, d_in] tensor")
    m, n = W.shape
    paths, outs = [], []
    for r in ranks:
        w = packed_words_per_row(r)
        p = dict(rank=int(r), u=torch.empty((m, w), dtype=torch.int32, device=W.device),
                 v=torch.empty((n, w), dtype=torch.int32, device=W.device),
                 h=torch.empty(m, dtype=torch.int16, device=W.device), g=torch.empty(n, dtype=torch.int16, device=W.device),
                 l=torch.empty(int(r), dtype=torch.int16, device=W.device))
        paths.append(p)
        outs.append(LbPathInit(int(r), p["u"].data_ptr(), p["v"].data_ptr(), p["h"].data_ptr(), p["g"].data_ptr(),
                               p["l"].data_ptr()))
    arr = (LbPathInit * len(outs))(*outs)
    _check(lib().lb_init_dual_svid(C.c_void_p(W.data_ptr()), m, n, arr, len(outs), _stream(stream)))
    return paths


def auto_regime(linears: Sequence["Linear"], tokens: int, io: int = BF16) -> int:
    """The regime LB_REGIME_AUTO runs for these linears at `tokens` tokens
    (lb_auto_regime)."""
    arr = (C.c_void_p * len(linears))(*[l.handle.value for l in linears])
    out = C.c_int()
    _check(lib().lb_auto_regime(arr, len(linears), int(tokens), int(io), C.byref(out)))
    return out.value


def _io_of(x, y) -> int:
    """lb_dtype of an (x, y) pair: both bf16, both fp32, or bf16 x with fp32 y."""
    import torch
    pair = (x.dtype, y.dtype)
    if pair == (torch.bfloat16, torch.bfloat16):
        return BF16
    if pair == (torch.float32, torch.float32):
        return FP32
    if pair == (torch.bfloat16, torch.float32):
        return BF16_FP32
    raise TypeError(f"x / y must be bf16 / bf16, fp32 / fp32 or bf16 / fp32, got {x.dtype} / {y.dtype}")


class Linear:
    """A factorised linear built by lb_linear_create from device tensors.

    ``paths`` is a list (1 or 2) of dicts with rank and device tensors
    u (int32 [d_out, W]), v (int32 [d_in, W]), h (int16/float16 [d_out]),
    g ([d_in]) and l ([rank]).
    """

    def __init__(self, d_out: int, d_in: int, paths: Sequence[Dict], stream=None):
        self.d_out, self.d_in = int(d_out), int(d_in)
        arr = (LbPath * max(1, len(paths)))()
        for i, p in enumerate(paths):
            arr[i].rank = int(p["rank"])
            arr[i].u_packed = p["u"].data_ptr()
            arr[i].v_packed = p["v"].data_ptr()
            arr[i].h = p["h"].data_ptr()
            arr[i].g = p["g"].data_ptr()
            arr[i].l = p["l"].data_ptr()
        h = C.c_void_p()
        _check(lib().lb_linear_create(self.d_out, self.d_in, arr, len(paths), _stream(stream), C.byref(h)))
        self.handle = h
        self.ranks = [int(p["rank"]) for p in paths]

    @classmethod
    def from_numpy(cls, d_out: int, d_in: int, paths: Sequence[Dict], device="cuda", stream=None):
        """Upload generator output (uint32 words, uint16 fp16 bits) and build the linear."""
        import torch
        dev = []
        for p in paths:
            dev.append(dict(
                rank=int(p["rank"]),
                u=torch.from_numpy(np.ascontiguousarray(p["u_words"]).view(np.int32)).to(device),
                v=torch.from_numpy(np.ascontiguousarray(p["v_words"]).view(np.int32)).to(device),
                h=torch.from_numpy(np.ascontiguousarray(p["h"]).view(np.int16)).to(device),
                g=torch.from_numpy(np.ascontiguousarray(p["g"]).view(np.int16)).to(device),
                l=torch.from_numpy(np.ascontiguousarray(p["l"]).view(np.int16)).to(device)))
        lin = cls(d_out, d_in, dev, stream=stream)
        torch.cuda.synchronize()  # the upload tensors may be freed after this
        return lin

    def info(self) -> Dict:
        m, n, dev = C.c_int64(), C.c_int64(), C.c_int64()
        npaths = C.c_int32()
        ranks = (C.c_int64 * 2)()
        _check(lib().lb_linear_info(self.handle, C.byref(m), C.byref(n), C.byref(npaths), ranks, C.byref(dev)))
        return dict(d_out=m.value, d_in=n.value, n_paths=npaths.value, ranks=list(ranks)[:npaths.value],
                    device_bytes=dev.value)

    def forward(self, x, y=None, regime: int = REGIME_AUTO, stream=None, out_dtype=None):
        """y = x W^T.  y (allocated when None, of out_dtype or x's dtype) sets
        the output type: bf16 x may write bf16 or fp32 y."""
        import torch
        if x.dim() != 2 or x.shape[1] != self.d_in:
            raise ValueError(f"x must be [tokens, {self.d_in}]")
        if not x.is_contiguous():
            raise ValueError("x must be contiguous")
        if not x.is_cuda:
            raise ValueError("x must be a device tensor")
        if y is None:
            y = torch.empty((x.shape[0], self.d_out), dtype=out_dtype or x.dtype, device=x.device)
        if y.dim() != 2 or tuple(y.shape) != (x.shape[0], self.d_out) or not y.is_contiguous():
            raise ValueError(f"y must be a contiguous [{x.shape[0]}, {self.d_out}] tensor")
        if y.device != x.device:
            raise ValueError("x and y must be on the same device")
        _check(lib().lb_linear_forward_ex(self.handle, x.data_ptr(), y.data_ptr(), x.shape[0], _io_of(x, y), regime,
                                          _stream(stream)))
        return y

    __call__ = forward

    def forward_noalloc(self, x, y, stream=None):
        """lb_linear_forward_noalloc: y = x W^T into the caller's y, with the
        library allocating nothing (decode kernels for bf16 x, exact kernels
        for fp32 I/O; its work buffers are the library's fixed scratch)."""
        if x.dim() != 2 or x.shape[1] != self.d_in or not x.is_contiguous() or not x.is_cuda:
            raise ValueError(f"x must be a contiguous device tensor [tokens, {self.d_in}]")
        if y.dim() != 2 or tuple(y.shape) != (x.shape[0], self.d_out) or not y.is_contiguous() or y.device != x.device:
            raise ValueError(f"y must be a contiguous [{x.shape[0]}, {self.d_out}] tensor on x's device")
        _check(lib().lb_linear_forward_noalloc(self.handle, x.data_ptr(), y.data_ptr(), x.shape[0], _io_of(x, y),
                                               _stream(stream)))
        return y

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().lb_linear_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Stack:
    """An ordered list of linears run together by lb_stack_forward."""

    def __init__(self, linears: Sequence[Linear]):
        self.linears = list(linears)
        arr = (C.c_void_p * len(self.linears))(*[l.handle.value for l in self.linears])
        h = C.c_void_p()
        _check(lib().lb_stack_create(arr, len(self.linears), C.byref(h)))
        self.handle = h

    def forward(self, xs: Sequence, ys: Sequence, regime: int = REGIME_AUTO, use_graph: Optional[bool] = None,
                stream=None):
        """use_graph None: the library's choice (lb_stack_forward); True / False:
        capture into a HIP graph and replay / launch directly."""
        n = len(self.linears)
        if len(xs) != n or len(ys) != n:
            raise ValueError("need one x and one y per linear")
        self.bind(xs, ys, regime, use_graph, stream).forward()
        return ys

    def bind(self, xs: Sequence, ys: Sequence, regime: int = REGIME_AUTO, use_graph: Optional[bool] = None,
             stream=None) -> "BoundStack":
        """The stack with its inputs, outputs, regime and stream fixed: the
        returned object's forward() passes the same pointer arrays each call
        (the per-call marshalling of hundreds of pointers otherwise costs more
        host time than a decode step takes on the GPU)."""
        return BoundStack(self, xs, ys, regime, use_graph, stream)

    __call__ = forward

    def set_persistent(self, mode) -> None:
        """lb_stack_set_persistent: run a chained decode's levels in one
        persistent launch (True or 1), as launches per level (False or 0, the
        default), or the persistent kernel's plans as launches per level (2,
        the same bits as 1)."""
        m = int(mode)
        if m not in (0, 1, 2):
            raise ValueError("mode must be 0, 1 or 2")
        _check(lib().lb_stack_set_persistent(self.handle, m))

    def persistent_status(self) -> Dict:
        """lb_stack_persistent_status: whether the current plan runs the
        persistent kernel, and whether a launch of it gave up (synchronises)."""
        active, aborted = C.c_int32(), C.c_int32()
        _check(lib().lb_stack_persistent_status(self.handle, C.byref(active), C.byref(aborted)))
        return dict(active=bool(active.value), aborted=bool(aborted.value))

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().lb_stack_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class BoundStack:
    """A Stack bound to fixed xs / ys (see Stack.bind).  It keeps references to
    the tensors, so their memory stays valid while it lives."""

    def __init__(self, stack: "Stack", xs: Sequence, ys: Sequence, regime: int, use_graph: Optional[bool], stream):
        n = len(stack.linears)
        if len(xs) != n or len(ys) != n:
            raise ValueError("need one x and one y per linear")
        pairs = {(x.dtype, y.dtype) for x, y in zip(xs, ys)}
        if len(pairs) != 1:
            raise TypeError("every entry of a stack forward must have the same x / y element types")
        tokens = int(xs[0].shape[0]) if xs[0].dim() == 2 else -1
        dev = xs[0].device
        # the library cannot see tensor shapes: a wrong-sized entry would be
        # read and written out of bounds on the device, so check each one here
        for i, (lin, x, y) in enumerate(zip(stack.linears, xs, ys)):
            if x.dim() != 2 or tuple(x.shape) != (tokens, lin.d_in):
                raise ValueError(f"entry {i}: x must be [{tokens}, {lin.d_in}], got {tuple(x.shape)}")
            if y.dim() != 2 or tuple(y.shape) != (tokens, lin.d_out):
                raise ValueError(f"entry {i}: y must be [{tokens}, {lin.d_out}], got {tuple(y.shape)}")
            if not x.is_contiguous() or not y.is_contiguous():
                raise ValueError(f"entry {i}: x and y must be contiguous")
        for i, (x, y) in enumerate(zip(xs, ys)):
            if not x.is_cuda or x.device != dev or y.device != dev:
                raise ValueError(f"entry {i}: every x and y must be on the same device ({dev})")
        self.stack, self.xs, self.ys = stack, list(xs), list(ys)
        self.tokens = tokens
        self.io = _io_of(xs[0], ys[0])
        self.xa = (C.c_void_p * n)(*[x.data_ptr() for x in xs])
        self.ya = (C.c_void_p * n)(*[y.data_ptr() for y in ys])
        self.regime = regime
        self.auto = use_graph is None and regime == REGIME_AUTO
        self.graph = 1 if (regime == REGIME_EXACT if use_graph is None else use_graph) else 0
        self.stream = _stream(stream)

    def forward(self):
        if self.auto:
            _check(lib().lb_stack_forward(self.stack.handle, self.xa, self.ya, self.tokens, self.io, self.stream))
        else:
            _check(lib().lb_stack_forward_ex(self.stack.handle, self.xa, self.ya, self.tokens, self.io, self.regime,
                                             self.graph, self.stream))
        return self.ys

    __call__ = forward
