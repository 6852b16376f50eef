"""fp32_reductions_amd -- Python binding of libreduce (gfx950 HIP kernels).

Thin ctypes layer over the C ABI in ``include/reduce.h``: it checks that
torch tensors have the dtype, device and extent an entry point expects,
passes their device pointers and the current HIP stream, and turns a
non-zero status into ``ReduceError``.  Every step of the reduction runs in
the HIP kernels of ``libreduce.so``; there is no CPU fallback.  Importing
this package raises if the library has not been built
(``python fp32_reductions_amd/build.py``).

Names follow the C ABI:

    sum_f32 / max_f32 / min_f32 (x, out, accum=False, stream=None)
    sum_max_min_f32 (x, out[3], accum=False, stream=None)
    sum_f32_atomic / max_f32_atomic / min_f32_atomic (same)
    sum_rows_f32 / max_rows_f32 / min_rows_f32 (x, out, n=None, accum=False)
    sum_cols_f32 / max_cols_f32 / min_cols_f32 (src, out, C=None, accum=False)
    colprod_f32 / colprod_f16 / colprod_bf16 / colprod_i32 (src, out, C=None)
    colprod_i16 / colprod_u16 / colprod_u32 (src, out, C=None)

``plan(name, *args, **kwargs)`` marshals the same arguments once and returns
a ``Plan``; calling it enqueues the C entry point with the stored pointers,
sizes and stream, without re-checking the tensors.  The caller keeps the
tensors alive and unchanged in shape while the plan is in use.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libreduce.so")

RED_OK, RED_ERR_INVALID, RED_ERR_ALIGN, RED_ERR_NOMEM, RED_ERR_HIP, RED_ERR_SCRATCH = range(6)


class ReduceError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_str(status), status))


if not os.path.exists(LIBRARY):
    raise ImportError(
        "libreduce.so is not built at %s; run "
        "'python fp32_reductions_amd/build.py' (hipcc, gfx950)" % LIBRARY)

_lib = ctypes.CDLL(LIBRARY)

_P, _SZ, _I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_SIGS = {
    "red_sum_f32": [_P, _SZ, _P, _I, _P],
    "red_max_f32": [_P, _SZ, _P, _I, _P],
    "red_min_f32": [_P, _SZ, _P, _I, _P],
    "red_sum_max_min_f32": [_P, _SZ, _P, _I, _P],
    "red_sum_max_min_f32_noalloc": [_P, _SZ, _P, _I, _P],
    "red_sum_f32_atomic": [_P, _SZ, _P, _I, _P],
    "red_max_f32_atomic": [_P, _SZ, _P, _I, _P],
    "red_min_f32_atomic": [_P, _SZ, _P, _I, _P],
    "red_sum_rows_f32": [_P, _SZ, _SZ, _SZ, _P, _I, _P],
    "red_max_rows_f32": [_P, _SZ, _SZ, _SZ, _P, _I, _P],
    "red_min_rows_f32": [_P, _SZ, _SZ, _SZ, _P, _I, _P],
    "red_sum_cols_f32": [_P, _SZ, _SZ, _SZ, _P, _I, _P],
    "red_max_cols_f32": [_P, _SZ, _SZ, _SZ, _P, _I, _P],
    "red_min_cols_f32": [_P, _SZ, _SZ, _SZ, _P, _I, _P],
    "red_colprod_f32": [_P, _SZ, _SZ, _SZ, _P, _P],
    "red_colprod_f16": [_P, _SZ, _SZ, _SZ, _P, _P],
    "red_colprod_bf16": [_P, _SZ, _SZ, _SZ, _P, _P],
    "red_colprod_i32": [_P, _SZ, _SZ, _SZ, _P, _P],
    "red_colprod_i16": [_P, _SZ, _SZ, _SZ, _P, _P],
    "red_colprod_u16": [_P, _SZ, _SZ, _SZ, _P, _P],
    "red_colprod_u32": [_P, _SZ, _SZ, _SZ, _P, _P],
    "red_release_workspace": [_P],
}
for _name, _args in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _I
_lib.red_status_str.argtypes = [_I]
_lib.red_status_str.restype = ctypes.c_char_p
_lib.red_abi_version.argtypes = []
_lib.red_abi_version.restype = _I

EXPORTS = tuple(_SIGS) + ("red_status_str", "red_abi_version")


def lib() -> ctypes.CDLL:
    """The loaded libreduce (raw C ABI, for callers holding raw pointers)."""
    return _lib


def status_str(status: int) -> str:
    return _lib.red_status_str(status).decode()


def abi_version() -> int:
    return _lib.red_abi_version()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def release_workspace(stream=None) -> None:
    """Free the library's workspace for `stream` (the current stream when
    None) after the work enqueued on it has finished."""
    _check(_lib.red_release_workspace(_stream(stream)), "red_release_workspace")


def _check(status: int, where: str) -> None:
    if status != RED_OK:
        raise ReduceError(status, where)


class Plan:
    """A C entry point with its arguments already marshalled."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name, args, keep):
        self.name = name
        self.fn = getattr(_lib, name)
        self.args = args
        self.keep = keep  # the tensors whose pointers are in args

    def __call__(self) -> None:
        status = self.fn(*self.args)
        if status != RED_OK:
            raise ReduceError(status, self.name)


def _need(t: torch.Tensor, dtype, what: str) -> None:
    """dtype may be one torch dtype or a tuple of accepted dtypes."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % what)
    ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
    if not ok:
        raise TypeError("%s must be %s, got %s" % (what, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be a device (cuda/HIP) tensor" % what)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)


# ---------------------------------------------------------------------------
# 1-D vector -> scalar
# ---------------------------------------------------------------------------

def _args_reduce1d(name: str, x, out, accum=False, stream=None):
    _need(x, torch.float32, "x")
    _need(out, torch.float32, "out")
    need = 3 if name.startswith("red_sum_max_min_f32") else 1
    if out.numel() < need:
        raise ValueError("out needs %d element(s)" % need)
    return (x.data_ptr(), x.numel(), out.data_ptr(), int(bool(accum)),
            _stream(stream)), (x, out)


def _reduce1d(name: str, x, out, accum, stream):
    args, _ = _args_reduce1d(name, x, out, accum, stream)
    _check(getattr(_lib, name)(*args), name)
    return out


def sum_f32(x, out, accum=False, stream=None):
    """out[0] = [out[0] +] sum(x), x any contiguous fp32 device tensor."""
    return _reduce1d("red_sum_f32", x, out, accum, stream)


def max_f32(x, out, accum=False, stream=None):
    return _reduce1d("red_max_f32", x, out, accum, stream)


def min_f32(x, out, accum=False, stream=None):
    return _reduce1d("red_min_f32", x, out, accum, stream)


def sum_max_min_f32(x, out, accum=False, stream=None):
    """out[0:3] = [out[0:3] (+, max, min)] (sum, max, min) of x, one read."""
    return _reduce1d("red_sum_max_min_f32", x, out, accum, stream)


def sum_max_min_f32_noalloc(x, out, accum=False, stream=None):
    """sum_max_min_f32 with its partials in the library's static scratch
    (no allocation); calls overlapping on one GPU race."""
    return _reduce1d("red_sum_max_min_f32_noalloc", x, out, accum, stream)


def sum_f32_atomic(x, out, accum=False, stream=None):
    return _reduce1d("red_sum_f32_atomic", x, out, accum, stream)


def max_f32_atomic(x, out, accum=False, stream=None):
    return _reduce1d("red_max_f32_atomic", x, out, accum, stream)


def min_f32_atomic(x, out, accum=False, stream=None):
    return _reduce1d("red_min_f32_atomic", x, out, accum, stream)


# ---------------------------------------------------------------------------
# segmented rows
# ---------------------------------------------------------------------------

def _args_rows(name: str, x, out, n=None, accum=False, stream=None):
    _need(x, torch.float32, "x")
    _need(out, torch.float32, "out")
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows, ld)")
    rows, ld = x.shape
    n = ld if n is None else int(n)
    if not 0 <= n <= ld:
        raise ValueError("need 0 <= n <= ld")
    if out.numel() < rows:
        raise ValueError("out needs one element per row")
    return (x.data_ptr(), rows, n, ld, out.data_ptr(), int(bool(accum)),
            _stream(stream)), (x, out)


def _rows(name: str, x, out, n, accum, stream):
    args, _ = _args_rows(name, x, out, n, accum, stream)
    _check(getattr(_lib, name)(*args), name)
    return out


def sum_rows_f32(x, out, n=None, accum=False, stream=None):
    """out[r] = [out[r] +] sum(x[r, :n]) for a row-major (rows, ld) x."""
    return _rows("red_sum_rows_f32", x, out, n, accum, stream)


def max_rows_f32(x, out, n=None, accum=False, stream=None):
    return _rows("red_max_rows_f32", x, out, n, accum, stream)


def min_rows_f32(x, out, n=None, accum=False, stream=None):
    return _rows("red_min_rows_f32", x, out, n, accum, stream)


# ---------------------------------------------------------------------------
# column sum / max / min
# ---------------------------------------------------------------------------

def _args_cols(name: str, src, out, C=None, accum=False, stream=None):
    _need(src, torch.float32, "src")
    _need(out, torch.float32, "out")
    if src.dim() != 2:
        raise ValueError("src must be 2-D (R, ld)")
    R, ld = src.shape
    C = ld if C is None else int(C)
    if not 0 <= C <= ld:
        raise ValueError("need 0 <= C <= ld")
    if out.numel() < C:
        raise ValueError("out needs C elements")
    return (src.data_ptr(), R, C, ld, out.data_ptr(), int(bool(accum)),
            _stream(stream)), (src, out)


def _cols(name: str, src, out, C, accum, stream):
    args, _ = _args_cols(name, src, out, C, accum, stream)
    _check(getattr(_lib, name)(*args), name)
    return out


def sum_cols_f32(src, out, C=None, accum=False, stream=None):
    """out[j] = [out[j] +] sum_i src[i, j] for j < C, fp32 (R, ld) tile."""
    return _cols("red_sum_cols_f32", src, out, C, accum, stream)


def max_cols_f32(src, out, C=None, accum=False, stream=None):
    return _cols("red_max_cols_f32", src, out, C, accum, stream)


def min_cols_f32(src, out, C=None, accum=False, stream=None):
    return _cols("red_min_cols_f32", src, out, C, accum, stream)


# ---------------------------------------------------------------------------
# column product
# ---------------------------------------------------------------------------

# Unsigned types may also arrive as the signed torch dtype of the same width
# (bit patterns): torch's uint16 / uint32 support on the device is partial.
_U16 = (torch.uint16, torch.int16) if hasattr(torch, "uint16") else (torch.int16,)
_U32 = (torch.uint32, torch.int32) if hasattr(torch, "uint32") else (torch.int32,)
_COLPROD_DTYPE = {"red_colprod_f32": torch.float32, "red_colprod_f16": torch.float16,
                  "red_colprod_bf16": torch.bfloat16, "red_colprod_i32": torch.int32,
                  "red_colprod_i16": torch.int16, "red_colprod_u16": _U16,
                  "red_colprod_u32": _U32}


def _args_colprod(name: str, src, out, C=None, stream=None):
    dtype = _COLPROD_DTYPE[name]
    _need(src, dtype, "src")
    _need(out, dtype, "out")
    if src.dim() != 2:
        raise ValueError("src must be 2-D (R, ld)")
    R, ld = src.shape
    C = ld if C is None else int(C)
    if not 0 <= C <= ld:
        raise ValueError("need 0 <= C <= ld")
    if out.numel() < C:
        raise ValueError("out needs C elements")
    return (src.data_ptr(), R, C, ld, out.data_ptr(), _stream(stream)), (src, out)


def _colprod(name: str, src, out, C, stream):
    args, _ = _args_colprod(name, src, out, C, stream)
    _check(getattr(_lib, name)(*args), name)
    return out


def colprod_f32(src, out, C=None, stream=None):
    """out[j] = prod_i src[i, j] for j < C (TCOLPROD), fp32."""
    return _colprod("red_colprod_f32", src, out, C, stream)


def colprod_f16(src, out, C=None, stream=None):
    """binary16 tile (torch.float16); fp32 products rounded once to fp16."""
    return _colprod("red_colprod_f16", src, out, C, stream)


def colprod_bf16(src, out, C=None, stream=None):
    """bfloat16 tile (torch.bfloat16); fp32 products rounded once to bf16."""
    return _colprod("red_colprod_bf16", src, out, C, stream)


def colprod_i32(src, out, C=None, stream=None):
    """int32 tile; products modulo 2^32."""
    return _colprod("red_colprod_i32", src, out, C, stream)


def colprod_i16(src, out, C=None, stream=None):
    """int16 tile; products modulo 2^16."""
    return _colprod("red_colprod_i16", src, out, C, stream)


def colprod_u16(src, out, C=None, stream=None):
    """uint16 tile (torch.uint16, or torch.int16 holding the bits); mod 2^16."""
    return _colprod("red_colprod_u16", src, out, C, stream)


def colprod_u32(src, out, C=None, stream=None):
    """uint32 tile (torch.uint32, or torch.int32 holding the bits); mod 2^32."""
    return _colprod("red_colprod_u32", src, out, C, stream)


# ---------------------------------------------------------------------------
# pre-marshalled calls
# ---------------------------------------------------------------------------

_MARSHAL = {}
for _op in ("sum", "max", "min"):
    _MARSHAL["%s_f32" % _op] = ("red_%s_f32" % _op, _args_reduce1d)
    _MARSHAL["%s_f32_atomic" % _op] = ("red_%s_f32_atomic" % _op, _args_reduce1d)
    _MARSHAL["%s_rows_f32" % _op] = ("red_%s_rows_f32" % _op, _args_rows)
    _MARSHAL["%s_cols_f32" % _op] = ("red_%s_cols_f32" % _op, _args_cols)
_MARSHAL["sum_max_min_f32"] = ("red_sum_max_min_f32", _args_reduce1d)
_MARSHAL["sum_max_min_f32_noalloc"] = ("red_sum_max_min_f32_noalloc", _args_reduce1d)
for _t in ("f32", "f16", "bf16", "i32", "i16", "u16", "u32"):
    _MARSHAL["colprod_" + _t] = ("red_colprod_" + _t, _args_colprod)


def plan(name: str, *args, **kwargs) -> Plan:
    """Marshal the arguments of entry point ``name`` (e.g. "sum_f32") once;
    the returned Plan enqueues the call each time it is called."""
    cname, marshal = _MARSHAL[name]
    cargs, keep = marshal(cname, *args, **kwargs)
    return Plan(cname, cargs, keep)
