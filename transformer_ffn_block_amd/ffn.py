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
VARIANTS = {"auto": 0, "fused": 1, "split": 2, "persistent": 3, "fused_norm": 4}

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
    ("ffn_swiglu_block_noalloc", _I, [_I, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _F, _I, _VP]),
    ("ffn_swiglu_block_persistent_status_offset", _SZ, [_I64, _I64, _I64]),
    ("ffn_swiglu_block_q8_workspace_size", _SZ, [_I64, _I64, _I64]),
    ("ffn_swiglu_block_q8", _I, [_VP, _VP, _Q8P, _Q8P, _Q8P, _VP, _I64, _I64, _I64, _F, _VP, _SZ, _VP]),
    ("ffn_swiglu_block_q4_workspace_size", _SZ, [_I64, _I64, _I64]),
    ("ffn_swiglu_block_q4", _I, [_VP, _VP, _Q4P, _Q4P, _Q4P, _VP, _I64, _I64, _I64, _F, _VP, _SZ, _VP]),
    ("ffn_status_string", ctypes.c_char_p, [_I]),
    ("ffn_last_error", ctypes.c_char_p, []),
    ("ffn_probe_read", _I, [_VP, _SZ, _VP, _I, _VP]),
    ("ffn_probe_read_groups", _I, [_I]),
    ("ffn_probe_copy", _I, [_VP, _VP, _SZ, _I, _I, _VP]),
    ("ffn_probe_mfma", _I, [_I, _I, _VP, _VP]),
    ("ffn_probe_mfma_groups", _I, [_I]),
    ("ffn_timing_enable", _I, [_I, _I]),
    ("ffn_timing_enabled", _I, []),
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


def _expect(t, name: str, shape, dtypes, device) -> None:
    """Raise ValueError unless t has exactly `shape`, one of `dtypes`, is
    contiguous and lives on `device` (checked before any library call, so a
    mismatched tensor never reaches the kernels as a raw pointer)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _expect_2d(x, name: str = "x"):
    if x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D [tokens, d] tensor, got shape {tuple(x.shape)}")
    return x.shape


def _workspace(workspace, need: int, device):
    if workspace is None:
        return alloc_workspace(need, device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.device != device:
        raise ValueError(f"workspace is on {workspace.device}, expected {device}")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise FFNError(FFN_ERR_WORKSPACE, "workspace", f"{nbytes} bytes given, {need} needed")
    return workspace


def _output(out, like, name="out"):
    torch = _torch()
    if out is None:
        return torch.empty_like(like)
    _expect(out, name, like.shape, (like.dtype,), like.device)
    return out


def _quant_operands(x, g, w_gate, w_up, w_down, qs_dtype, nibbles: bool):
    """Check a quantised block's operands: x [M,d] and g [d] bf16, each
    weight a (qs, scales) pair with qs [N, K] (Q8_0, int8) or [N, K/2]
    (Q4_0, uint8) and scales [N, K/32] 16-bit fp16 patterns."""
    torch = _torch()
    M, d = _expect_2d(x)
    _expect(x, "x", (M, d), (torch.bfloat16,), x.device)
    _expect(g, "g", (d,), (torch.bfloat16,), x.device)
    for name, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        if not isinstance(w, (tuple, list)) or len(w) != 2:
            raise ValueError(f"{name} must be a (qs, scales) pair")
    if w_gate[0].dim() != 2:
        raise ValueError(f"w_gate quants must be 2-D, got shape {tuple(w_gate[0].shape)}")
    f = w_gate[0].shape[0]
    for name, (qs, sc), N, K in (("w_gate", w_gate, f, d), ("w_up", w_up, f, d), ("w_down", w_down, d, f)):
        if K % 32 or N <= 0:
            raise ValueError(f"{name}: the reduction length {K} must be a positive multiple of 32")
        _expect(qs, f"{name} quants", (N, K // 2 if nibbles else K), (qs_dtype,), x.device)
        _expect(sc, f"{name} scales", (N, K // 32), (torch.int16, torch.uint16), x.device)
    return M, d, f


def rmsnorm(x, g, eps: float, out=None, stream=None):
    """y = rmsnorm(x) * g over the last dim of a [rows, d] tensor."""
    rows, d = _expect_2d(x)
    _dt(x)
    _expect(g, "g", (d,), (x.dtype,), x.device)
    y = _output(out, x)
    check(lib().ffn_rmsnorm(_dt(x), _dev(x, "x"), _dev(g, "g"), _dev(y, "y"), rows, d, eps,
                            _stream_handle(stream)), "ffn_rmsnorm")
    return y


def workspace_size(dtype_code: int, M: int, d: int, f: int, variant: str = "auto") -> int:
    return lib().ffn_swiglu_block_workspace_size(dtype_code, M, d, f, VARIANTS[variant])


def alloc_workspace(nbytes: int, device="cuda"):
    """A device byte buffer for the workspace (torch allocations are 256-byte aligned)."""
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _block_operands(x, g, w_gate, w_up, w_down):
    M, d = _expect_2d(x)
    dt = _dt(x)
    if w_gate.dim() != 2:
        raise ValueError(f"w_gate must be a 2-D [f, d] tensor, got shape {tuple(w_gate.shape)}")
    f = w_gate.shape[0]
    _expect(g, "g", (d,), (x.dtype,), x.device)
    _expect(w_gate, "w_gate", (f, d), (x.dtype,), x.device)
    _expect(w_up, "w_up", (f, d), (x.dtype,), x.device)
    _expect(w_down, "w_down", (d, f), (x.dtype,), x.device)
    return M, d, f, dt


def swiglu_block(x, g, w_gate, w_up, w_down, eps: float, variant: str = "auto", out=None,
                 workspace=None, stream=None, check_status: bool = True):
    """y = x + W_down (silu(W_gate n) * (W_up n)), n = rmsnorm(x) * g.

    variant "persistent" has bounded device-side waits; with check_status
    (the default) the call synchronises the stream and raises FFNError if a
    wait gave up (the result is then wrong).  Timing loops pass
    check_status=False and read persistent_status() themselves."""
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}; choose from {sorted(VARIANTS)}")
    M, d, f, dt = _block_operands(x, g, w_gate, w_up, w_down)
    need = workspace_size(dt, M, d, f, variant)
    ws = _workspace(workspace, need, x.device)
    y = _output(out, x)
    check(lib().ffn_swiglu_block(dt, _dev(x, "x"), _dev(g, "g"), _dev(w_gate, "w_gate"),
                                 _dev(w_up, "w_up"), _dev(w_down, "w_down"), _dev(y, "y"), M, d, f,
                                 eps, VARIANTS[variant], ws.data_ptr(), ws.numel() * ws.element_size(),
                                 _stream_handle(stream)), "ffn_swiglu_block")
    if variant == "persistent" and check_status and M > 0:
        (stream if stream is not None else _torch().cuda.current_stream()).synchronize()
        word = persistent_status(ws, M, d, f)
        if word != 0:
            raise FFNError(FFN_ERR_LAUNCH, "ffn_swiglu_block(persistent)",
                           f"a work item gave up waiting (error word {word:#x}); the result is invalid")
    return y


def swiglu_block_noalloc(x, g, w_gate, w_up, w_down, eps: float, variant: str = "auto", out=None,
                         stream=None):
    """The block with the library's own scratch array as its workspace (no
    device allocation by the library; `out` preallocated by the caller for
    the same guarantee on this side).  Calls that overlap on one GPU race."""
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}; choose from {sorted(VARIANTS)}")
    M, d, f, dt = _block_operands(x, g, w_gate, w_up, w_down)
    y = _output(out, x)
    check(lib().ffn_swiglu_block_noalloc(dt, _dev(x, "x"), _dev(g, "g"), _dev(w_gate, "w_gate"),
                                         _dev(w_up, "w_up"), _dev(w_down, "w_down"), _dev(y, "y"),
                                         M, d, f, eps, VARIANTS[variant], _stream_handle(stream)),
          "ffn_swiglu_block_noalloc")
    return y


def persistent_status(workspace, M: int, d: int, f: int) -> int:
    """The error word a completed PERSISTENT call left in its workspace (0 = ok).
    Reads device memory: call after the call's stream has been synchronised."""
    off = lib().ffn_swiglu_block_persistent_status_offset(M, d, f)
    if off == 0:
        raise ValueError(f"no persistent schedule for M={M}, d={d}, f={f}")
    b = workspace.view(-1)[off:off + 4].to("cpu").numpy()
    return int(b.view("<u4")[0])


def q8_struct(qs, scales) -> Q8Matrix:
    return Q8Matrix(_dev(qs, "qs"), _dev(scales, "scales"))


def swiglu_block_q8(x, g, w_gate: Tuple, w_up: Tuple, w_down: Tuple, eps: float, out=None,
                    workspace=None, stream=None):
    """The block with Q8_0 weights; each weight is a (qs int8 [N,K], scales int16/uint16-bits [N,K/32]) pair."""
    torch = _torch()
    M, d, f = _quant_operands(x, g, w_gate, w_up, w_down, torch.int8, nibbles=False)
    need = lib().ffn_swiglu_block_q8_workspace_size(M, d, f)
    ws = _workspace(workspace, need, x.device)
    y = _output(out, x)
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
    M, d, f = _quant_operands(x, g, w_gate, w_up, w_down, torch.uint8, nibbles=True)
    need = lib().ffn_swiglu_block_q4_workspace_size(M, d, f)
    ws = _workspace(workspace, need, x.device)
    y = _output(out, x)
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
    torch = _torch()
    if kind not in ("q8", "q4"):
        raise ValueError(f"kind must be 'q8' or 'q4', got {kind!r}")
    M, d, f = _quant_operands(x, g, w_gate, w_up, w_down, torch.int8 if kind == "q8" else torch.uint8,
                              nibbles=kind == "q4")
    _output(out, x)
    L = lib()
    need = getattr(L, f"ffn_swiglu_block_{kind}_workspace_size")(M, d, f)
    _workspace(workspace, need, x.device)
    nbytes = workspace.numel() * workspace.element_size()
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


def probe_copy(src, dst, groups_per_cu: int = 0, nontemporal: bool = False, stream=None) -> None:
    if src.numel() * src.element_size() != dst.numel() * dst.element_size():
        raise ValueError("probe_copy: src and dst must have the same size in bytes")
    check(lib().ffn_probe_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(),
                               groups_per_cu, 1 if nontemporal else 0, _stream_handle(stream)),
          "ffn_probe_copy")


def probe_mfma(iters: int, waves_per_cu: int, sink, stream=None) -> int:
    """Run the matrix-core loop; returns the flop it executes."""
    groups = lib().ffn_probe_mfma_groups(waves_per_cu)
    if sink.numel() * sink.element_size() < 4 * 256 * groups:
        raise ValueError("probe_mfma: sink too small")
    check(lib().ffn_probe_mfma(iters, waves_per_cu, sink.data_ptr(), _stream_handle(stream)),
          "ffn_probe_mfma")
    return groups * 4 * 8 * iters * 16384


def timing_enable(on: bool, max_launches: int = 4096) -> None:
    check(lib().ffn_timing_enable(1 if on else 0, max_launches), "ffn_timing_enable")


def timing_enabled() -> bool:
    """Whether per-kernel timing is on for the calling thread."""
    return bool(lib().ffn_timing_enabled())


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
