"""CPU oracle for the CSA/HCA Compressor (THD gated-softmax pooling).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``gated_pooling_amd``) never imports it and the C code here shares nothing
with the HIP library.

The arithmetic lives in ``csa_oracle.c`` (plain C, built with gcc as
``liboracle.so``); this module only marshals numpy arrays.  bf16 tensors are
passed as their uint16 bit patterns.

Functions (see ``csa_oracle.c`` for the definitions and their sources):
  total_comp(cu, r)                       -> N = sum_s floor(L_s / r)
  exp_f32(y)                              -> the fixed fp32 exponential
  fwd_f32(kv, score, ape, cu, T, r, c, d) -> out bf16 bits [N, d]
  bwd_f32(..., dout)                      -> dkv, dscore bf16 bits, dape f64, ds32, o32
  fwd_f64(kv, score, ape64, cu, T, r, c, d) -> out f64 [N, d]
  bwd_f64(..., dout)                      -> dkv, dscore, dape (f64)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = [
    "-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
]


def build(force: bool = True) -> str:
    """Compile csa_oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_exp_f32.restype = ctypes.c_float
        L.oracle_exp_f32.argtypes = [ctypes.c_float]
        L.oracle_exp_f32_array.restype = None
        L.oracle_exp_f32_array.argtypes = [P, P, i64]
        L.oracle_exp_constants.restype = None
        L.oracle_exp_constants.argtypes = [P]
        L.oracle_bf16_from_f32.restype = ctypes.c_uint16
        L.oracle_bf16_from_f32.argtypes = [ctypes.c_float]
        L.oracle_f32_from_bf16.restype = ctypes.c_float
        L.oracle_f32_from_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_total_comp.restype = ctypes.c_int
        L.oracle_total_comp.argtypes = [P, i32, i32, P]
        L.oracle_fwd_f32.restype = ctypes.c_int
        L.oracle_fwd_f32.argtypes = [P, P, P, P, i32, i64, i32, i32, i32, P, i64]
        L.oracle_bwd_f32.restype = ctypes.c_int
        L.oracle_bwd_f32.argtypes = [P, P, P, P, i32, i64, i32, i32, i32, P, i64, P, P, P, P, P]
        L.oracle_fwd_f64.restype = ctypes.c_int
        L.oracle_fwd_f64.argtypes = [P, P, P, P, i32, i64, i32, i32, i32, P, i64]
        L.oracle_bwd_f64.restype = ctypes.c_int
        L.oracle_bwd_f64.argtypes = [P, P, P, P, i32, i64, i32, i32, i32, P, i64, P, P, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of later oracle calls."""
    lib().oracle_set_num_threads(int(n))


def total_comp(cu, r: int) -> int:
    cu = _c(cu, np.int32)
    out = np.zeros(1, np.int64)
    _check(lib().oracle_total_comp(_ptr(cu), len(cu) - 1, r, _ptr(out)), "total_comp")
    return int(out[0])


def exp_f32(y: float) -> float:
    return float(np.float32(lib().oracle_exp_f32(float(np.float32(y)))))


def exp_f32_array(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty_like(y)
    lib().oracle_exp_f32_array(_ptr(y), _ptr(out), y.size)
    return out


def exp_constants() -> np.ndarray:
    out = np.zeros(12, np.float32)
    lib().oracle_exp_constants(_ptr(out))
    return out


def bf16_from_f32(x: float) -> int:
    return int(lib().oracle_bf16_from_f32(float(np.float32(x))))


def f32_from_bf16(h: int) -> float:
    return float(lib().oracle_f32_from_bf16(int(h)))


def f64_from_bits(bits) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16 array)."""
    b = _c(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fwd_f32(kv, score, ape, cu, T_cap: int, r: int, c: int, d: int, out=None) -> np.ndarray:
    kv, score = _c(kv, np.uint16), _c(score, np.uint16)
    ape, cu = _c(ape, np.float32), _c(cu, np.int32)
    N = total_comp(cu, r)
    if out is None:
        out = np.full((N, d), 0x7FC0, np.uint16)
    _check(lib().oracle_fwd_f32(_ptr(kv), _ptr(score), _ptr(ape), _ptr(cu), len(cu) - 1,
                                T_cap, r, c, d, _ptr(out), N), "fwd_f32")
    return out


def bwd_outputs(T_cap: int, r: int, c: int, d: int, N: int):
    """NaN-prefilled output arrays for bwd_f32 (a slot the oracle forgot to
    write stays visible).  Reusable across calls of the same shape."""
    W = c * d
    return (np.full((T_cap, W), 0x7FC0, np.uint16), np.full((T_cap, W), 0x7FC0, np.uint16),
            np.full((r, W), np.nan, np.float64), np.full((T_cap, W), np.nan, np.float32),
            np.full((N, d), np.nan, np.float32))


def bwd_f32(kv, score, ape, cu, T_cap: int, r: int, c: int, d: int, dout, outs=None):
    """Returns (dkv bits, dscore bits, dape f64, ds32 f32, o32 f32).  `outs`
    may pass arrays from bwd_outputs() to avoid reallocating."""
    kv, score = _c(kv, np.uint16), _c(score, np.uint16)
    ape, cu, dout = _c(ape, np.float32), _c(cu, np.int32), _c(dout, np.uint16)
    N = total_comp(cu, r)
    dkv, dscore, dape, ds32, o32 = outs if outs is not None else bwd_outputs(T_cap, r, c, d, N)
    _check(lib().oracle_bwd_f32(_ptr(kv), _ptr(score), _ptr(ape), _ptr(cu), len(cu) - 1,
                                T_cap, r, c, d, _ptr(dout), N, _ptr(dkv), _ptr(dscore),
                                _ptr(dape), _ptr(ds32), _ptr(o32)), "bwd_f32")
    return dkv, dscore, dape, ds32, o32


def fwd_f64(kv, score, ape, cu, T_cap: int, r: int, c: int, d: int) -> np.ndarray:
    """kv, score, ape: float64 values (widen bf16 inputs with f64_from_bits)."""
    kv, score = _c(kv, np.float64), _c(score, np.float64)
    ape, cu = _c(ape, np.float64), _c(cu, np.int32)
    N = total_comp(cu, r)
    out = np.full((N, d), np.nan, np.float64)
    _check(lib().oracle_fwd_f64(_ptr(kv), _ptr(score), _ptr(ape), _ptr(cu), len(cu) - 1,
                                T_cap, r, c, d, _ptr(out), N), "fwd_f64")
    return out


def bwd_f64(kv, score, ape, cu, T_cap: int, r: int, c: int, d: int, dout):
    """float64 inputs (dout too); returns (dkv, dscore, dape) in float64."""
    kv, score = _c(kv, np.float64), _c(score, np.float64)
    ape, cu, dout = _c(ape, np.float64), _c(cu, np.int32), _c(dout, np.float64)
    N = total_comp(cu, r)
    W = c * d
    dkv = np.full((T_cap, W), np.nan, np.float64)
    dscore = np.full((T_cap, W), np.nan, np.float64)
    dape = np.full((r, W), np.nan, np.float64)
    _check(lib().oracle_bwd_f64(_ptr(kv), _ptr(score), _ptr(ape), _ptr(cu), len(cu) - 1,
                                T_cap, r, c, d, _ptr(dout), N, _ptr(dkv), _ptr(dscore),
                                _ptr(dape)), "bwd_f64")
    return dkv, dscore, dape
