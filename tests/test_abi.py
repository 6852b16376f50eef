"""The C ABI without a GPU: the library loads, exports every function that
include/reduce.h declares, and rejects invalid arguments (or accepts empty
input) before it makes any HIP call.

No call here can reach a kernel launch: every call either has empty input
(returns before any HIP call) or fails validation.  Pointers are fake
integers that are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "reduce.h")
LIBRARY = os.path.join(ROOT, "fp32_reductions_amd", "libreduce.so")

RED_OK, RED_ERR_INVALID, RED_ERR_ALIGN, RED_ERR_NOMEM, RED_ERR_HIP, RED_ERR_SCRATCH = range(6)

# Fake device addresses: aligned and misaligned; never dereferenced.
A16 = 0x7F0000000000
P = ctypes.c_void_p
SZ = ctypes.c_size_t
I = ctypes.c_int


def declared_functions():
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(red_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIBRARY):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_libreduce_build", os.path.join(ROOT, "fp32_reductions_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return ctypes.CDLL(LIBRARY)


def test_header_declares_the_abi():
    names = declared_functions()
    for op in ("sum", "max", "min"):
        assert "red_%s_f32" % op in names
        assert "red_%s_f32_atomic" % op in names
        assert "red_%s_rows_f32" % op in names
        assert "red_%s_cols_f32" % op in names
    assert "red_sum_max_min_f32" in names
    for t in ("f32", "f16", "bf16", "i32", "i16", "u16", "u32"):
        assert "red_colprod_" + t in names
    assert "red_status_str" in names and "red_abi_version" in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIBRARY],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (red_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        getattr(lib, n)  # resolvable through the dynamic loader


def test_version_and_status_strings(lib):
    lib.red_abi_version.restype = I
    with open(HEADER) as fh:
        ver = int(re.search(r"#define RED_ABI_VERSION (\d+)", fh.read()).group(1))
    assert lib.red_abi_version() == ver
    lib.red_status_str.restype = ctypes.c_char_p
    lib.red_status_str.argtypes = [I]
    texts = [lib.red_status_str(s).decode() for s in range(6)]
    assert texts[0] == "ok" and len(set(texts)) == 6
    assert lib.red_status_str(99).decode() == "unknown status"


def _fn(lib, name, argtypes):
    f = getattr(lib, name)
    f.argtypes = argtypes
    f.restype = I
    return f


@pytest.mark.parametrize("name", ["red_sum_f32", "red_max_f32", "red_min_f32",
                                  "red_sum_max_min_f32", "red_sum_max_min_f32_noalloc",
                                  "red_sum_f32_atomic", "red_max_f32_atomic",
                                  "red_min_f32_atomic"])
def test_1d_validation(lib, name):
    f = _fn(lib, name, [P, SZ, P, I, P])
    # empty input: OK, even with null pointers and accum
    assert f(None, 0, None, 1, None) == RED_OK
    assert f(A16, 0, A16, 0, None) == RED_OK
    # null pointers for non-empty input
    assert f(None, 5, A16, 0, None) == RED_ERR_INVALID
    assert f(A16, 5, None, 1, None) == RED_ERR_INVALID
    # element count whose byte size overflows
    assert f(A16, (1 << 63), A16, 0, None) == RED_ERR_INVALID
    # pointers not 4-byte aligned
    assert f(A16 + 2, 5, A16, 0, None) == RED_ERR_ALIGN
    assert f(A16, 5, A16 + 1, 0, None) == RED_ERR_ALIGN


@pytest.mark.parametrize("name", ["red_sum_rows_f32", "red_max_rows_f32",
                                  "red_min_rows_f32"])
def test_rows_validation(lib, name):
    f = _fn(lib, name, [P, SZ, SZ, SZ, P, I, P])
    assert f(None, 0, 10, 10, None, 1, None) == RED_OK      # rows == 0
    assert f(None, 10, 0, 10, None, 1, None) == RED_OK      # n == 0
    assert f(None, 3, 4, 4, A16, 0, None) == RED_ERR_INVALID
    assert f(A16, 3, 4, 4, None, 0, None) == RED_ERR_INVALID
    assert f(A16, 3, 5, 4, A16, 0, None) == RED_ERR_INVALID  # ld < n
    assert f(A16, 1 << 40, 1 << 30, 1 << 30, A16, 0, None) == RED_ERR_INVALID
    assert f(A16 + 2, 3, 4, 4, A16, 0, None) == RED_ERR_ALIGN
    assert f(A16, 3, 4, 4, A16 + 3, 0, None) == RED_ERR_ALIGN


@pytest.mark.parametrize("name", ["red_sum_cols_f32", "red_max_cols_f32",
                                  "red_min_cols_f32"])
def test_cols_validation(lib, name):
    f = _fn(lib, name, [P, SZ, SZ, SZ, P, I, P])
    assert f(None, 0, 16, 16, None, 1, None) == RED_OK
    assert f(None, 16, 0, 16, None, 1, None) == RED_OK
    assert f(None, 4, 4, 4, A16, 0, None) == RED_ERR_INVALID
    assert f(A16, 4, 4, 4, None, 0, None) == RED_ERR_INVALID
    assert f(A16, 4, 5, 4, A16, 0, None) == RED_ERR_INVALID      # ld < C
    assert f(A16, 1 << 40, 1 << 30, 1 << 30, A16, 0, None) == RED_ERR_INVALID
    assert f(A16, 1, 1 << 30, 1 << 30, A16, 0, None) == RED_ERR_INVALID  # 2^24 column blocks
    assert f(A16 + 2, 4, 4, 4, A16, 0, None) == RED_ERR_ALIGN
    assert f(A16, 4, 4, 4, A16 + 1, 0, None) == RED_ERR_ALIGN


@pytest.mark.parametrize("name,es", [("red_colprod_f32", 4), ("red_colprod_i32", 4),
                                     ("red_colprod_f16", 2), ("red_colprod_bf16", 2),
                                     ("red_colprod_i16", 2), ("red_colprod_u16", 2),
                                     ("red_colprod_u32", 4)])
def test_colprod_validation(lib, name, es):
    f = _fn(lib, name, [P, SZ, SZ, SZ, P, P])
    # TCOLPROD's early return: zero valid rows or columns
    assert f(None, 0, 16, 16, None, None) == RED_OK
    assert f(None, 16, 0, 16, None, None) == RED_OK
    assert f(None, 4, 4, 4, A16, None) == RED_ERR_INVALID
    assert f(A16, 4, 4, 4, None, None) == RED_ERR_INVALID
    assert f(A16, 4, 5, 4, A16, None) == RED_ERR_INVALID      # ld < C
    assert f(A16, 1 << 40, 1 << 30, 1 << 30, A16, None) == RED_ERR_INVALID
    assert f(A16, 2, 1 << 40, 1 << 40, A16, None) == RED_ERR_INVALID  # grid limit
    # exactly 2^24 column blocks of 16 lanes x 16 bytes: one too many
    C = (1 << 24) * 16 * (16 // es)
    assert f(A16, 1, C, C, A16, None) == RED_ERR_INVALID
    assert f(A16 + 1, 4, 4, 4, A16, None) == RED_ERR_ALIGN
    assert f(A16, 4, 4, 4, A16 + 1, None) == RED_ERR_ALIGN
    if es == 4:
        assert f(A16 + 2, 4, 4, 4, A16, None) == RED_ERR_ALIGN
