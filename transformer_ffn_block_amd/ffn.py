"""Thin ctypes binding of libffn.so (the C ABI in include/ffn.h).

Argument marshalling only: every step of the block runs in the library's
HIP kernels.  torch provides device memory (outputs, workspaces) and the
current stream.  Loading fails loudly if the library is missing; there is
no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libffn.so")

FFN_OK, FFN_ERR_INVALID_ARGUMENT, FFN_ERR_UNSUPPORTED, FFN_ERR_WORKSPACE, FFN_ERR_LAUNCH = range(5)
FFN_F32, FFN_BF16 = 0, 1
VARIANTS = {"auto": 0, "fused": 1, "split": 2, "persistent": 3}

# (name, restype, argtypes) of every function include/ffn.h declares
_VP, _I64, _F, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t


class Q8Matrix(ctypes.Structure):
    _fields_ = [("qs", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Q4Matrix(ctypes.Structure):
    _fields_ = [("qs", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_Q8P = ctypes.POINTER(Q8Matrix)
_Q4P = ctypes.POINTER(Q4Matrix)
SIGNATURES = [
    ("ffn_rmsnorm", _I, [_I, _VP, _VP, _VP, _I64, _I64, _F, _VP]),
    ("ffn_swiglu_block_workspace_size", _SZ, [_I, _I64, _I64, _I64, _I]),
    ("ffn_swiglu_block", _I, [_I, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _F, _I, _VP, _SZ, _VP]),
    ("ffn_swiglu_block_q8_workspace_size", _SZ, [_I64, _I64, _I64]),
    ("ffn_swiglu_block_q8", _I, [_VP, _VP, _Q8P, _Q8P, _Q8P, _VP, _I64, _I64, _I64, _F, _VP, _SZ, _VP]),
    ("ffn_swiglu_block_q4_workspace_size", _SZ, [_I64, _I64, _I64]),
    ("ffn_swiglu_block_q4", _I, [_VP, _VP, _Q4P, _Q4P, _Q4P, _VP, _I64, _I64, _I64, _F, _VP, _SZ, _VP]),
    ("ffn_status_string", ctypes.c_char_p, [_I]),
    ("ffn_last_error", ctypes.c_char_p, []),
    ("ffn_probe_read", _I, [_VP, _SZ, _VP, _I, _VP]),
    ("ffn_probe_read_groups", _I, [_I]),
    ("ffn_probe_copy", _I, [_VP, _VP, _SZ, _VP]),
    ("ffn_timing_enable", _I, [_I, _I]),
    ("ffn_timing_collect", _I, []),
    ("ffn_timing_count", _I, []),
    ("ffn_timing_get", _I, [_I, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_I64),
                            ctypes.POINTER(ctypes.c_double)]),
    ("ffn_timing_reset", None, []),
]

_lib: Optional[ctypes.CDLL] = None


class FFNError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({_status_name(status)}): {detail}")


_NAMES = ["FFN_OK", "FFN_ERR_INVALID_ARGUMENT", "FFN_ERR_UNSUPPORTED", "FFN_ERR_WORKSPACE", "FFN_ERR_LAUNCH"]


def _status_name(s: int) -> str:
    return _NAMES[s] if 0 <= s < len(_NAMES) else "FFN_ERR_UNKNOWN"


def lib() -> ctypes.CDLL:
    """Load libffn.so (in-tree) once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m transformer_ffn_block_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int, where: str) -> None:
    if status != FFN_OK:
        raise FFNError(status, where, lib().ffn_last_error().decode())


# ----------------------------------------------------------------------------
# torch-tensor level helpers (torch only supplies memory and the stream)
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_handle(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FFN_BF16
    if t.dtype == torch.float32:
        return FFN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def rmsnorm(x, g, eps: float, out=None, stream=None):
    """y = rmsnorm(x) * g over the last dim of a [rows, d] tensor."""
    torch = _torch()
    rows, d = x.shape
    y = out if out is not None else torch.empty_like(x)
    check(lib().ffn_rmsnorm(_dt(x), _dev(x, "x"), _dev(g, "g"), _dev(y, "y"), rows, d, eps,
                            _stream_handle(stream)), "ffn_rmsnorm")
    return y


def workspace_size(dtype_code: int, M: int, d: int, f: int, variant: str = "auto") -> int:
    return lib().ffn_swiglu_block_workspace_size(dtype_code, M, d, f, VARIANTS[variant])


def alloc_workspace(nbytes: int, device="cuda"):
    """A device byte buffer for the workspace (torch allocations are 256-byte aligned)."""
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def swiglu_block(x, g, w_gate, w_up, w_down, eps: float, variant: str = "auto", out=None,
                 workspace=None, stream=None):
    """y = x + W_down (silu(W_gate n) * (W_up n)), n = rmsnorm(x) * g."""
    torch = _torch()
    M, d = x.shape
    f = w_gate.shape[0]
    dt = _dt(x)
    need = workspace_size(dt, M, d, f, variant)
    ws = workspace if workspace is not None else alloc_workspace(need, x.device)
    y = out if out is not None else torch.empty_like(x)
    check(lib().ffn_swiglu_block(dt, _dev(x, "x"), _dev(g, "g"), _dev(w_gate, "w_gate"),
                                 _dev(w_up, "w_up"), _dev(w_down, "w_down"), _dev(y, "y"), M, d, f,
                                 eps, VARIANTS[variant], ws.data_ptr(), ws.numel() * ws.element_size(),
                                 _stream_handle(stream)), "ffn_swiglu_block")
    return y


def q8_struct(qs, scales) -> Q8Matrix:
    return Q8Matrix(_dev(qs, "qs"), _dev(scales, "scales"))


def swiglu_block_q8(x, g, w_gate: Tuple, w_up: Tuple, w_down: Tuple, eps: float, out=None,
                    workspace=None, stream=None):
    """The block with Q8_0 weights; each weight is a (qs int8 [N,K], scales int16/uint16-bits [N,K/32]) pair."""
    torch = _torch()
    M, d = x.shape
    f = w_gate[0].shape[0]
    need = lib().ffn_swiglu_block_q8_workspace_size(M, d, f)
    ws = workspace if workspace is not None else alloc_workspace(need, x.device)
    y = out if out is not None else torch.empty_like(x)
    mg, mu, md = q8_struct(*w_gate), q8_struct(*w_up), q8_struct(*w_down)
    check(lib().ffn_swiglu_block_q8(_dev(x, "x"), _dev(g, "g"), ctypes.byref(mg), ctypes.byref(mu),
                                    ctypes.byref(md), _dev(y, "y"), M, d, f, eps, ws.data_ptr(),
                                    ws.numel() * ws.element_size(), _stream_handle(stream)),
          "ffn_swiglu_block_q8")
    return y


def q4_struct(qs, scales) -> Q4Matrix:
    return Q4Matrix(_dev(qs, "qs"), _dev(scales, "scales"))


def swiglu_block_q4(x, g, w_gate: Tuple, w_up: Tuple, w_down: Tuple, eps: float, out=None,
                    workspace=None, stream=None):
    """The block with Q4_0 weights; each weight is a (qs uint8 [N,K/2], scales int16/uint16-bits [N,K/32]) pair."""
    torch = _torch()
    M, d = x.shape
    f = w_gate[0].shape[0]
    need = lib().ffn_swiglu_block_q4_workspace_size(M, d, f)
    ws = workspace if workspace is not None else alloc_workspace(need, x.device)
    y = out if out is not None else torch.empty_like(x)
    mg, mu, md = q4_struct(*w_gate), q4_struct(*w_up), q4_struct(*w_down)
    check(lib().ffn_swiglu_block_q4(_dev(x, "x"), _dev(g, "g"), ctypes.byref(mg), ctypes.byref(mu),
                                    ctypes.byref(md), _dev(y, "y"), M, d, f, eps, ws.data_ptr(),
                                    ws.numel() * ws.element_size(), _stream_handle(stream)),
          "ffn_swiglu_block_q4")
    return y


def prepare_swiglu_block_quant(kind: str, x, g, w_gate: Tuple, w_up: Tuple, w_down: Tuple,
                               eps: float, out, workspace, stream=None):
    """Marshal one ffn_swiglu_block_q8 / _q4 call (kind "q8" / "q4") once and
    return a function that issues it and checks its status.  For loops that
    repeat the same call (timing): the weight structs and pointers are built
    here, not per call.  The tensors must stay alive and unchanged in place."""
    M, d = x.shape
    f = w_gate[0].shape[0]
    L = lib()
    need = getattr(L, f"ffn_swiglu_block_{kind}_workspace_size")(M, d, f)
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise FFNError(FFN_ERR_WORKSPACE, f"ffn_swiglu_block_{kind}", f"workspace {nbytes} < {need} bytes")
    mk = q8_struct if kind == "q8" else q4_struct
    mats = [mk(*w) for w in (w_gate, w_up, w_down)]
    fn = getattr(L, f"ffn_swiglu_block_{kind}")
    args = (_dev(x, "x"), _dev(g, "g"), *[ctypes.byref(m) for m in mats], _dev(out, "y"), M, d, f, eps,
            workspace.data_ptr(), nbytes, _stream_handle(stream))

    def call():
        st = fn(*args)
        if st:
            check(st, f"ffn_swiglu_block_{kind}")
    call.mats = mats  # keeps the structs alive with the closure
    return call


# ----------------------------------------------------------------------------
# measurement helpers
# ----------------------------------------------------------------------------
def probe_read(src, sink, waves_per_cu: int, stream=None) -> None:
    check(lib().ffn_probe_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                               waves_per_cu, _stream_handle(stream)), "ffn_probe_read")


def probe_copy(src, dst, stream=None) -> None:
    check(lib().ffn_probe_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(),
                               _stream_handle(stream)), "ffn_probe_copy")


def timing_enable(on: bool, max_launches: int = 4096) -> None:
    check(lib().ffn_timing_enable(1 if on else 0, max_launches), "ffn_timing_enable")


def timing_collect() -> dict:
    """Wait for the recorded per-kernel events; return {kernel: (launches, total_ms)} so far."""
    L = lib()
    check(L.ffn_timing_collect(), "ffn_timing_collect")
    out = {}
    for i in range(L.ffn_timing_count()):
        name = ctypes.c_char_p()
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        check(L.ffn_timing_get(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)), "ffn_timing_get")
        out[name.value.decode()] = (n.value, ms.value)
    return out


def timing_reset() -> None:
    lib().ffn_timing_reset()


def exported_symbols() -> Sequence[str]:
    return [s[0] for s in SIGNATURES]
