"""Plain CPU oracle for dense-array reduction -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP
library in ``fp32_reductions_amd`` and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, built with
gcc and no fast-math); this module only builds it, loads it with ctypes and
moves numpy arrays in and out.  What each function computes, and the page
passage it follows, is stated in ``oracle.c``:

* sum / max / min of a 1-D fp32 vector, with accum -- TVM TIRx docs,
  "reduction -> sm100_packed" (introduction; "How inputs change the
  algorithm");
* the page's own single-precision summation order -- same page, "Algorithm";
* column sum / max / min of a 2-D fp32 tile -- the same reduction along rows;
* column products over fp32 / fp16 / bf16 / int16 / uint16 / int32 / uint32
  -- PTO ISA "TCOLPROD"
  ("Math Interpretation", "Constraints").
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

# Strict IEEE: no fast-math, no fused multiply-add contraction.
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
          "-fPIC", "-shared", "-pthread"]


def source_digest(source: str = SOURCE) -> str:
    """SHA-256 of the C source and the compiler flags it is built with."""
    h = hashlib.sha256()
    with open(source, "rb") as fh:
        h.update(fh.read())
    h.update(" ".join(CFLAGS).encode())
    return h.hexdigest()


def _stamp(library: str) -> str:
    return library + ".sha256"


def build(source: str = SOURCE, library: str = LIBRARY) -> str:
    """Compile ``source`` with gcc into ``library``; returns the library path.
    The digest of the source is recorded beside the library."""
    tmp = library + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, source, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, library)
    with open(_stamp(library) + ".tmp%d" % os.getpid(), "w") as fh:
        fh.write(source_digest(source) + "\n")
    os.replace(_stamp(library) + ".tmp%d" % os.getpid(), _stamp(library))
    return library


def ensure_built(source: str = SOURCE, library: str = LIBRARY) -> str:
    """The library, rebuilt first when it is missing or was built from a
    different source (its recorded digest differs from the source's)."""
    try:
        with open(_stamp(library)) as fh:
            recorded = fh.read().strip()
    except OSError:
        recorded = None
    if not os.path.exists(library) or recorded != source_digest(source):
        build(source, library)
    return library


_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I = ctypes.c_int


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class Oracle:
    """ctypes view of one build of ``oracle.c``."""

    def __init__(self, library: str = LIBRARY):
        lib = ctypes.CDLL(library)
        sig = {
            "oracle_sum_f32": [_P, _SZ, _I, ctypes.c_float, _P, _P],
            "oracle_max_f32": [_P, _SZ, _I, _P],
            "oracle_min_f32": [_P, _SZ, _I, _P],
            "oracle_page_sum_f32": [_P, _SZ, _I, _P],
            "oracle_rows_sum_f32": [_P, _SZ, _SZ, _SZ, _I, _P, _P, _P],
            "oracle_rows_max_f32": [_P, _SZ, _SZ, _SZ, _I, _P],
            "oracle_rows_min_f32": [_P, _SZ, _SZ, _SZ, _I, _P],
            "oracle_rows_page_sum_f32": [_P, _SZ, _SZ, _SZ, _I, _P],
            "oracle_colprod_f32": [_P, _SZ, _SZ, _SZ, _P],
            "oracle_colprod_f16": [_P, _SZ, _SZ, _SZ, _P],
            "oracle_colprod_bf16": [_P, _SZ, _SZ, _SZ, _P],
            "oracle_colprod_i32": [_P, _SZ, _SZ, _SZ, _P],
            "oracle_colprod_u32": [_P, _SZ, _SZ, _SZ, _P],
            "oracle_colprod_u16": [_P, _SZ, _SZ, _SZ, _P],
            "oracle_cols_sum_f32": [_P, _SZ, _SZ, _SZ, _I, _P, _P, _P],
            "oracle_cols_max_f32": [_P, _SZ, _SZ, _SZ, _I, _P],
            "oracle_cols_min_f32": [_P, _SZ, _SZ, _SZ, _I, _P],
            "oracle_sum_f32_mt": [_P, _SZ, _I, ctypes.c_float, _I, _P, _P],
            "oracle_max_f32_mt": [_P, _SZ, _I, _I, _P],
            "oracle_min_f32_mt": [_P, _SZ, _I, _I, _P],
            "oracle_rows_sum_f32_mt": [_P, _SZ, _SZ, _SZ, _I, _P, _P],
            "oracle_rows_max_f32_mt": [_P, _SZ, _SZ, _SZ, _I, _P],
            "oracle_colprod_f32_mt": [_P, _SZ, _SZ, _SZ, _I, _P],
            "oracle_colprod_f16_mt": [_P, _SZ, _SZ, _SZ, _I, _P],
            "oracle_colprod_bf16_mt": [_P, _SZ, _SZ, _SZ, _I, _P],
            "oracle_colprod_i32_mt": [_P, _SZ, _SZ, _SZ, _I, _P],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _I
        for name in ("oracle_f16_to_f64", "oracle_bf16_to_f64"):
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_uint16]
            fn.restype = ctypes.c_double
        self.lib = lib

    # -- 1-D ------------------------------------------------------------
    def sum_f32(self, x, accum: bool = False, old: float = 0.0):
        """(S, A): the exact-as-possible sum (fp64) and the sum of |terms|.
        None when x is empty (nothing is computed, as for an empty tile)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        s = np.zeros(1, np.float64)
        a = np.zeros(1, np.float64)
        ok = self.lib.oracle_sum_f32(_ptr(x), x.size, int(bool(accum)),
                                     float(old), _ptr(s), _ptr(a))
        return (float(s[0]), float(a[0])) if ok else None

    def _extreme(self, fn, x, accum, old):
        x = np.ascontiguousarray(x, dtype=np.float32)
        d = np.array([old], dtype=np.float32)
        fn(_ptr(x), x.size, int(bool(accum)), _ptr(d))
        return d[0]

    def max_f32(self, x, accum: bool = False, old: float = 0.0) -> np.float32:
        """maxNum over x (and old under accum); returns old for empty x."""
        return self._extreme(self.lib.oracle_max_f32, x, accum, old)

    def min_f32(self, x, accum: bool = False, old: float = 0.0) -> np.float32:
        return self._extreme(self.lib.oracle_min_f32, x, accum, old)

    def page_sum_f32(self, x, accum: bool = False, old: float = 0.0) -> np.float32:
        """The page's 8-slot single-precision order (returns old if empty)."""
        return self._extreme(self.lib.oracle_page_sum_f32, x, accum, old)

    # -- rows -----------------------------------------------------------
    @staticmethod
    def _rows_view(x, rows, n, ld):
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        if rows and n:
            assert x.size >= (rows - 1) * ld + n, "buffer too small"
        return x

    def rows_sum_f32(self, x, rows, n, ld, accum=False, old=None):
        """Per-row (S, A) arrays in fp64; None for an empty problem."""
        x = self._rows_view(x, rows, n, ld)
        o = (np.zeros(rows, np.float32) if old is None
             else np.ascontiguousarray(old, dtype=np.float32))
        s = np.zeros(rows, np.float64)
        a = np.zeros(rows, np.float64)
        ok = self.lib.oracle_rows_sum_f32(_ptr(x), rows, n, ld,
                                          int(bool(accum)), _ptr(o),
                                          _ptr(s), _ptr(a))
        return (s, a) if ok else None

    def _rows_inplace(self, fn, x, rows, n, ld, accum, dst):
        x = self._rows_view(x, rows, n, ld)
        d = (np.zeros(rows, np.float32) if dst is None
             else np.array(dst, dtype=np.float32, copy=True))
        fn(_ptr(x), rows, n, ld, int(bool(accum)), _ptr(d))
        return d

    def rows_max_f32(self, x, rows, n, ld, accum=False, dst=None):
        return self._rows_inplace(self.lib.oracle_rows_max_f32, x, rows, n,
                                  ld, accum, dst)

    def rows_min_f32(self, x, rows, n, ld, accum=False, dst=None):
        return self._rows_inplace(self.lib.oracle_rows_min_f32, x, rows, n,
                                  ld, accum, dst)

    def rows_page_sum_f32(self, x, rows, n, ld, accum=False, dst=None):
        return self._rows_inplace(self.lib.oracle_rows_page_sum_f32, x, rows,
                                  n, ld, accum, dst)

    # -- colprod --------------------------------------------------------
    def _colprod(self, fn, src, R, C, ld, dtype, out_dtype, dst):
        src = np.ascontiguousarray(src).reshape(-1)
        assert src.dtype == dtype, (src.dtype, dtype)
        if R and C:
            assert src.size >= (R - 1) * ld + C, "buffer too small"
        d = (np.zeros(C, out_dtype) if dst is None
             else np.array(dst, dtype=out_dtype, copy=True))
        fn(_ptr(src), R, C, ld, _ptr(d))
        return d

    def colprod_f32(self, src, R, C, ld, dst=None):
        """fp64 column products of an fp32 tile (dst untouched if R*C == 0)."""
        return self._colprod(self.lib.oracle_colprod_f32, src, R, C, ld,
                             np.float32, np.float64, dst)

    def colprod_f16(self, src_bits, R, C, ld, dst=None):
        """fp64 column products of a binary16 tile given as uint16 bits."""
        return self._colprod(self.lib.oracle_colprod_f16, src_bits, R, C, ld,
                             np.uint16, np.float64, dst)

    def colprod_bf16(self, src_bits, R, C, ld, dst=None):
        """fp64 column products of a bfloat16 tile given as uint16 bits."""
        return self._colprod(self.lib.oracle_colprod_bf16, src_bits, R, C, ld,
                             np.uint16, np.float64, dst)

    def colprod_i32(self, src, R, C, ld, dst=None):
        """int32 column products modulo 2^32."""
        return self._colprod(self.lib.oracle_colprod_i32, src, R, C, ld,
                             np.int32, np.int32, dst)

    def colprod_u32(self, src, R, C, ld, dst=None):
        """uint32 column products modulo 2^32."""
        return self._colprod(self.lib.oracle_colprod_u32, src, R, C, ld,
                             np.uint32, np.uint32, dst)

    def colprod_u16(self, src_bits, R, C, ld, dst=None):
        """int16 / uint16 column products modulo 2^16, as uint16 patterns."""
        return self._colprod(self.lib.oracle_colprod_u16, src_bits, R, C, ld,
                             np.uint16, np.uint16, dst)

    # -- column sum / max / min -----------------------------------------
    def cols_sum_f32(self, src, R, C, ld, accum=False, old=None):
        """Per-column (S, A) arrays in fp64; None for an empty tile."""
        src = self._rows_view(src, R, C, ld)
        o = (np.zeros(C, np.float32) if old is None
             else np.ascontiguousarray(old, dtype=np.float32))
        s = np.zeros(C, np.float64)
        a = np.zeros(C, np.float64)
        ok = self.lib.oracle_cols_sum_f32(_ptr(src), R, C, ld, int(bool(accum)),
                                          _ptr(o), _ptr(s), _ptr(a))
        return (s, a) if ok else None

    def cols_max_f32(self, src, R, C, ld, accum=False, dst=None):
        return self._cols_inplace(self.lib.oracle_cols_max_f32, src, R, C, ld,
                                  accum, dst)

    def cols_min_f32(self, src, R, C, ld, accum=False, dst=None):
        return self._cols_inplace(self.lib.oracle_cols_min_f32, src, R, C, ld,
                                  accum, dst)

    def _cols_inplace(self, fn, src, R, C, ld, accum, dst):
        src = self._rows_view(src, R, C, ld)
        d = (np.zeros(C, np.float32) if dst is None
             else np.array(dst, dtype=np.float32, copy=True))
        fn(_ptr(src), R, C, ld, int(bool(accum)), _ptr(d))
        return d

    # -- threaded forms (timing on several host cores) -------------------
    @staticmethod
    def _mt_status(rc):
        if rc < 0:
            raise RuntimeError("oracle: could not start its threads")
        return rc

    def sum_f32_mt(self, x, threads: int, accum: bool = False, old: float = 0.0):
        """sum_f32 over `threads` contiguous pieces, combined in order."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        s = np.zeros(1, np.float64)
        a = np.zeros(1, np.float64)
        ok = self._mt_status(self.lib.oracle_sum_f32_mt(
            _ptr(x), x.size, int(bool(accum)), float(old), int(threads), _ptr(s), _ptr(a)))
        return (float(s[0]), float(a[0])) if ok else None

    def _extreme_mt(self, fn, x, threads, accum, old):
        x = np.ascontiguousarray(x, dtype=np.float32)
        d = np.array([old], dtype=np.float32)
        self._mt_status(fn(_ptr(x), x.size, int(bool(accum)), int(threads), _ptr(d)))
        return d[0]

    def max_f32_mt(self, x, threads: int, accum: bool = False, old: float = 0.0):
        return self._extreme_mt(self.lib.oracle_max_f32_mt, x, threads, accum, old)

    def min_f32_mt(self, x, threads: int, accum: bool = False, old: float = 0.0):
        return self._extreme_mt(self.lib.oracle_min_f32_mt, x, threads, accum, old)

    def rows_sum_f32_mt(self, x, rows, n, ld, threads: int):
        x = self._rows_view(x, rows, n, ld)
        s = np.zeros(rows, np.float64)
        a = np.zeros(rows, np.float64)
        ok = self._mt_status(self.lib.oracle_rows_sum_f32_mt(
            _ptr(x), rows, n, ld, int(threads), _ptr(s), _ptr(a)))
        return (s, a) if ok else None

    def rows_max_f32_mt(self, x, rows, n, ld, threads: int):
        x = self._rows_view(x, rows, n, ld)
        d = np.zeros(rows, np.float32)
        self._mt_status(self.lib.oracle_rows_max_f32_mt(_ptr(x), rows, n, ld, int(threads),
                                                        _ptr(d)))
        return d

    def _colprod_mt(self, fn, src, R, C, ld, dtype, out_dtype, threads):
        src = np.ascontiguousarray(src).reshape(-1)
        assert src.dtype == dtype, (src.dtype, dtype)
        if R and C:
            assert src.size >= (R - 1) * ld + C, "buffer too small"
        d = np.zeros(C, out_dtype)
        self._mt_status(fn(_ptr(src), R, C, ld, int(threads), _ptr(d)))
        return d

    def colprod_f32_mt(self, src, R, C, ld, threads: int):
        return self._colprod_mt(self.lib.oracle_colprod_f32_mt, src, R, C, ld,
                                np.float32, np.float64, threads)

    def colprod_f16_mt(self, src_bits, R, C, ld, threads: int):
        return self._colprod_mt(self.lib.oracle_colprod_f16_mt, src_bits, R, C, ld,
                                np.uint16, np.float64, threads)

    def colprod_bf16_mt(self, src_bits, R, C, ld, threads: int):
        return self._colprod_mt(self.lib.oracle_colprod_bf16_mt, src_bits, R, C, ld,
                                np.uint16, np.float64, threads)

    def colprod_i32_mt(self, src, R, C, ld, threads: int):
        return self._colprod_mt(self.lib.oracle_colprod_i32_mt, src, R, C, ld,
                                np.int32, np.int32, threads)

    def f16_to_f64(self, h: int) -> float:
        return self.lib.oracle_f16_to_f64(h)

    def bf16_to_f64(self, b: int) -> float:
        return self.lib.oracle_bf16_to_f64(b)


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from the current ``oracle.c`` (compiled on first use
    when the library is absent or was built from another source)."""
    global _default
    if _default is None:
        _default = Oracle(ensure_built())
    return _default
