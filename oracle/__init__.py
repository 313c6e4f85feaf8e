"""CPU oracle for C = A * B (fp64 accumulation, own decoders, own RNE rounding).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The library
under ``invariant_matmul_amd`` never imports it and shares no code with it;
the two meet only through the seeded input generators in ``workloads``.

Every function here works on raw bit patterns (numpy ``uint8``/``uint16``
arrays) so that both sides consume the very same input bytes.  The arithmetic
lives in ``oracle.c``; this module only builds it and marshals arguments.

Pins (the tests that tie the oracle to something other than itself):
decoders are checked exhaustively against torch's own conversions; the RNE
helper against the binary16 worked example of the Tencent article on
deterministic inference (section "背景": 2048 + 1 rounds to 2048, the next
value after 2048 is 2050) and against torch/numpy casts; the product against
closed forms (identity, all-ones giving K, unit selectors, zeros), an int64
brute-force twin, exactly-representable "grid" inputs and numpy's fp64 matmul
within its error bound.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FORMATS = {"f16": 0, "bf16": 1, "e4m3": 2, "e5m2": 3, "f32": 4}
_BITS_DTYPE = {"f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8,
               "e5m2": np.uint8, "f32": np.uint32}

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def bind(lib):
    """Declare the C signatures on a loaded copy of the oracle library."""
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
    lib.orc_decode.argtypes = [ctypes.c_int, vp, i64, vp]
    lib.orc_round.argtypes = [ctypes.c_int, vp, i64, vp]
    lib.orc_gemm.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp, dp, vp, vp, ctypes.c_int]
    lib.orc_gemm_rows.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp, dp, vp, i64,
                                  vp, vp, ctypes.c_int]
    lib.orc_gemm_elems.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp, dp, vp, vp, i64,
                                   vp, vp, ctypes.c_int]
    lib.orc_gemm_i64.argtypes = [i64, i64, i64, vp, vp, vp]
    for f in ("orc_decode", "orc_round", "orc_gemm", "orc_gemm_rows", "orc_gemm_elems",
              "orc_gemm_i64", "orc_max_threads"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = bind(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _bits(fmt: str, x) -> np.ndarray:
    a = np.ascontiguousarray(x)
    want = _BITS_DTYPE[fmt]
    if a.dtype != want:
        if a.dtype.itemsize != np.dtype(want).itemsize:
            raise TypeError(f"{fmt} bit patterns must be {np.dtype(want).name}, got {a.dtype}")
        a = a.view(want)
    return a


def decode(fmt: str, bits) -> np.ndarray:
    """Exact fp64 values of the bit patterns ``bits`` in format ``fmt``."""
    b = _bits(fmt, bits)
    out = np.empty(b.shape, dtype=np.float64)
    rc = _load().orc_decode(FORMATS[fmt], _ptr(b), b.size, _ptr(out))
    if rc:
        raise ValueError(f"orc_decode({fmt}) failed: {rc}")
    return out


def round_rne(fmt: str, x) -> np.ndarray:
    """Bit patterns of ``x`` (fp64) rounded to ``fmt`` with ties to even."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=_BITS_DTYPE[fmt])
    rc = _load().orc_round(FORMATS[fmt], _ptr(a), a.size, _ptr(out))
    if rc:
        raise ValueError(f"orc_round({fmt}) failed: {rc}")
    return out


def gemm(A_bits, B_bits, fmt: str, scale: float = 1.0, rows=None, nthreads: int = 0):
    """(C64, Cabs) for C = scale * A @ B, with A [M,K] and B [K,N] as bit patterns.

    ``C64`` is the fp64 ascending-k sum (unrounded), ``Cabs`` is
    ``|scale| * |A| @ |B|`` for the error bound.  With ``rows`` given, only
    those rows of A are evaluated and the outputs have ``len(rows)`` rows.
    """
    A = _bits(fmt, A_bits)
    B = _bits(fmt, B_bits)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch {A.shape} @ {B.shape}")
    M, K = A.shape
    N = B.shape[1]
    lib = _load()
    if rows is None:
        C = np.empty((M, N), dtype=np.float64)
        Ca = np.empty((M, N), dtype=np.float64)
        rc = lib.orc_gemm(M, N, K, FORMATS[fmt], _ptr(A), _ptr(B), float(scale),
                          _ptr(C), _ptr(Ca), int(nthreads))
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        C = np.empty((r.size, N), dtype=np.float64)
        Ca = np.empty((r.size, N), dtype=np.float64)
        rc = lib.orc_gemm_rows(M, N, K, FORMATS[fmt], _ptr(A), _ptr(B), float(scale),
                               _ptr(r), r.size, _ptr(C), _ptr(Ca), int(nthreads))
    if rc:
        raise ValueError(f"orc_gemm failed: {rc}")
    return C, Ca


def linear(x_bits, w_bits, fmt: str, bias=None, scale: float = 1.0, rows=None,
           nthreads: int = 0):
    """(Y64, Yabs) for the linear layer Y = scale * x @ W^T + bias.

    The layer a batch-invariant inference stack puts on top of the matrix
    product (the vLLM batch-invariant ``linear`` operator listed in the
    closing section of the Tencent deterministic-inference article): x is
    [M, K], the weight W is [N, K] (one row per output feature), bias is an
    fp64-decodable vector of N values or None.  ``Y64`` is the exact product
    from ``gemm`` (with B = W^T) plus the bias, added in fp64; ``Yabs`` is
    ``|scale| |x| |W^T| + |bias|`` for the error bound.
    """
    W = _bits(fmt, w_bits)
    if W.ndim != 2:
        raise ValueError(f"weight must be 2-D, got {W.shape}")
    C, Ca = gemm(x_bits, np.ascontiguousarray(W.T), fmt, scale=scale, rows=rows,
                 nthreads=nthreads)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)
        if b.shape != (C.shape[1],):
            raise ValueError(f"bias must have {C.shape[1]} values, got {b.shape}")
        C = C + b[None, :]
        Ca = Ca + np.abs(b)[None, :]
    return C, Ca


def gemm_elems(A_bits, B_bits, fmt: str, ii, jj, scale: float = 1.0, nthreads: int = 0):
    """(c64, cabs) at the listed output positions (ii[t], jj[t])."""
    A = _bits(fmt, A_bits)
    B = _bits(fmt, B_bits)
    M, K = A.shape
    N = B.shape[1]
    if B.shape[0] != K:
        raise ValueError(f"shape mismatch {A.shape} @ {B.shape}")
    i = np.ascontiguousarray(ii, dtype=np.int64)
    j = np.ascontiguousarray(jj, dtype=np.int64)
    if i.shape != j.shape:
        raise ValueError("ii and jj must have the same length")
    c = np.empty(i.size, dtype=np.float64)
    ca = np.empty(i.size, dtype=np.float64)
    rc = _load().orc_gemm_elems(M, N, K, FORMATS[fmt], _ptr(A), _ptr(B), float(scale),
                                _ptr(i), _ptr(j), i.size, _ptr(c), _ptr(ca), int(nthreads))
    if rc:
        raise ValueError(f"orc_gemm_elems failed: {rc}")
    return c, ca


def gemm_i64(A_int, B_int) -> np.ndarray:
    """Integer twin: A @ B in int64 by the plain triple loop (int32 inputs)."""
    A = np.ascontiguousarray(A_int, dtype=np.int32)
    B = np.ascontiguousarray(B_int, dtype=np.int32)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch {A.shape} @ {B.shape}")
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), dtype=np.int64)
    rc = _load().orc_gemm_i64(M, N, K, _ptr(A), _ptr(B), _ptr(C))
    if rc:
        raise ValueError(f"orc_gemm_i64 failed: {rc}")
    return C


def max_threads() -> int:
    """Threads the fp64 loops use by default (OpenMP's current maximum)."""
    return int(_load().orc_max_threads())
