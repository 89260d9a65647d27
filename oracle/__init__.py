"""CPU oracle for dense half-precision GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding in ``dense_half_precision_amd``) never imports it; the two share
no code.

The arithmetic lives in ``hgemm_oracle.c`` (plain C, FP64 accumulation,
IEEE round-to-nearest-even written from the format definitions).  This module
builds it with gcc and wraps it with ctypes over numpy ``uint16`` bit
patterns, so the same host bits that feed the GPU feed the oracle.

Definition: ``ref[m, n] = RNE_dtype(sum_k A[m, k] * Bop[k, n])`` with the sum in
FP64, ``Bop = Bt.T`` for TN and ``B`` for NN -- the naive matmul of the
"tcgen05 for dummies" translation (recap section) with the TN/NN layouts of
the "HGEMM: WMMA 与 MMA PTX 代码学习" kernel header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hgemm_oracle.c")

F16, BF16 = 0, 1
TN, NN = 0, 1
_DTYPES = {"f16": F16, "fp16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16}
_LAYOUTS = {"tn": TN, "nn": NN}


def lib_path(mutation: int = 0) -> str:
    name = "liboracle.so" if mutation == 0 else f"liboracle_mut{mutation}.so"
    return os.path.join(_HERE, name)


def build(mutation: int = 0, force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math).  Returns the .so path."""
    out = lib_path(mutation)
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           f"-DORACLE_MUTATION={mutation}", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_LIBS: dict[int, ctypes.CDLL] = {}


def _load(mutation: int = 0) -> ctypes.CDLL:
    if mutation in _LIBS:
        return _LIBS[mutation]
    path = build(mutation, force=False)
    lib = ctypes.CDLL(path)
    i64, u16p, f64p, i64p = (ctypes.c_int64, ctypes.POINTER(ctypes.c_uint16),
                             ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64))
    lib.oracle_decode_array.argtypes = [ctypes.c_int, u16p, f64p, i64]
    lib.oracle_round_array.argtypes = [ctypes.c_int, f64p, u16p, i64]
    lib.oracle_hgemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, u16p, u16p, u16p]
    lib.oracle_hgemm.restype = ctypes.c_int
    lib.oracle_hgemm_rows.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, u16p, u16p,
                                      u16p, i64, i64]
    lib.oracle_hgemm_rows.restype = ctypes.c_int
    lib.oracle_hgemm_sampled.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, u16p, u16p,
                                         i64p, i64p, i64, u16p]
    lib.oracle_hgemm_sampled.restype = ctypes.c_int
    dbl = ctypes.c_double
    lib.oracle_gemm_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64, dbl,
                                     u16p, i64, u16p, i64, dbl, u16p, i64, u16p, i64, i64, i64]
    lib.oracle_gemm_rows.restype = ctypes.c_int
    lib.oracle_gemm_sampled.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                        dbl, u16p, i64, u16p, i64, dbl, u16p, i64, i64p, i64p,
                                        i64, u16p]
    lib.oracle_gemm_sampled.restype = ctypes.c_int
    lib.oracle_mutation.restype = ctypes.c_int
    _LIBS[mutation] = lib
    return lib


def _code(table: dict, key) -> int:
    if isinstance(key, int):
        return key
    return table[str(key).lower()]


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {a.dtype}")
    return a


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def decode(bits: np.ndarray, dtype, mutation: int = 0) -> np.ndarray:
    """Exact values (float64) of 16-bit patterns of the given dtype."""
    b = _u16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load(mutation).oracle_decode_array(_code(_DTYPES, dtype), _ptr(b, ctypes.c_uint16),
                                        _ptr(out, ctypes.c_double), b.size)
    return out


def round_to(x: np.ndarray, dtype, mutation: int = 0) -> np.ndarray:
    """Round float64 values to the dtype (RNE); returns uint16 bit patterns."""
    xx = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(xx.shape, dtype=np.uint16)
    _load(mutation).oracle_round_array(_code(_DTYPES, dtype), _ptr(xx, ctypes.c_double),
                                       _ptr(out, ctypes.c_uint16), xx.size)
    return out


def _shapes(layout: int, A: np.ndarray, B: np.ndarray):
    M, K = A.shape
    if layout == TN:
        N, K2 = B.shape
    else:
        K2, N = B.shape
    if K2 != K:
        raise ValueError(f"K mismatch: A has {K}, B has {K2}")
    return M, N, K


def hgemm(layout, dtype, A: np.ndarray, B: np.ndarray, mutation: int = 0,
          rows: tuple[int, int] | None = None) -> np.ndarray:
    """Full reference output (uint16 bits, shape [M, N]).

    ``layout`` is "tn" (B holds Bt[N, K]) or "nn" (B holds B[K, N]).
    With ``rows=(r0, r1)`` only that band is computed; other rows are zero.
    """
    lay = _code(_LAYOUTS, layout)
    A, B = _u16(A), _u16(B)
    M, N, K = _shapes(lay, A, B)
    C = np.zeros((M, N), dtype=np.uint16)
    r0, r1 = rows if rows is not None else (0, M)
    rc = _load(mutation).oracle_hgemm_rows(lay, _code(_DTYPES, dtype), M, N, K,
                                           _ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16),
                                           _ptr(C, ctypes.c_uint16), r0, r1)
    if rc != 0:
        raise RuntimeError(f"oracle_hgemm failed with {rc}")
    return C


def hgemm_sampled(layout, dtype, A: np.ndarray, B: np.ndarray, rows: np.ndarray,
                  cols: np.ndarray, mutation: int = 0) -> np.ndarray:
    """Reference values at (rows[i], cols[i]) (uint16 bits)."""
    lay = _code(_LAYOUTS, layout)
    A, B = _u16(A), _u16(B)
    M, N, K = _shapes(lay, A, B)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(r.shape, dtype=np.uint16)
    rc = _load(mutation).oracle_hgemm_sampled(lay, _code(_DTYPES, dtype), M, N, K,
                                              _ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16),
                                              _ptr(r, ctypes.c_int64), _ptr(c, ctypes.c_int64),
                                              r.size, _ptr(out, ctypes.c_uint16))
    if rc != 0:
        raise RuntimeError(f"oracle_hgemm_sampled failed with {rc}")
    return out


# ------------------------------------------------------------------ general form
def _gen_check(opA: int, opB: int, M: int, N: int, K: int, A, B, beta, Cin):
    if opA not in (0, 1) or opB not in (0, 1):
        raise ValueError("opA/opB must be 0 (as stored) or 1 (transposed)")
    ra, ca = (M, K) if opA == 0 else (K, M)
    rb, cb = (K, N) if opB == 0 else (N, K)
    if A.ndim != 2 or A.shape[0] < ra or A.shape[1] < ca:
        raise ValueError(f"A stored as {A.shape} cannot hold {ra} x {ca}")
    if B.ndim != 2 or B.shape[0] < rb or B.shape[1] < cb:
        raise ValueError(f"B stored as {B.shape} cannot hold {rb} x {cb}")
    if beta != 0 and (Cin is None or Cin.ndim != 2 or Cin.shape[0] < M or Cin.shape[1] < N):
        raise ValueError("beta != 0 needs Cin of at least M x N")


def gemm(opA: int, opB: int, dtype, M: int, N: int, K: int, A: np.ndarray, B: np.ndarray,
         alpha: float = 1.0, beta: float = 0.0, Cin: np.ndarray | None = None,
         mutation: int = 0, rows: tuple[int, int] | None = None) -> np.ndarray:
    """General form ``C = RNE(alpha * opA(A) opB(B) + beta * Cin)`` (uint16 bits, M x N).

    A, B and Cin are 2-D uint16 arrays in their stored shape; the length of a
    stored row is that operand's leading dimension (opA 0: A is M x K, 1: A is
    stored K x M; opB 0: B is K x N, 1: B is stored N x K).  With beta == 0
    Cin is not read.
    """
    A, B = _u16(A), _u16(B)
    _gen_check(opA, opB, M, N, K, A, B, beta, Cin)
    cin = _u16(Cin) if (Cin is not None and beta != 0) else None
    C = np.zeros((M, N), dtype=np.uint16)
    r0, r1 = rows if rows is not None else (0, M)
    rc = _load(mutation).oracle_gemm_rows(
        opA, opB, _code(_DTYPES, dtype), M, N, K, float(alpha), _ptr(A, ctypes.c_uint16),
        A.shape[1], _ptr(B, ctypes.c_uint16), B.shape[1], float(beta),
        _ptr(cin, ctypes.c_uint16) if cin is not None else None,
        cin.shape[1] if cin is not None else 0, _ptr(C, ctypes.c_uint16), N, r0, r1)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_rows failed with {rc}")
    return C


def gemm_sampled(opA: int, opB: int, dtype, M: int, N: int, K: int, A: np.ndarray,
                 B: np.ndarray, rows: np.ndarray, cols: np.ndarray, alpha: float = 1.0,
                 beta: float = 0.0, Cin: np.ndarray | None = None,
                 mutation: int = 0) -> np.ndarray:
    """General form at (rows[i], cols[i]) (uint16 bits)."""
    A, B = _u16(A), _u16(B)
    _gen_check(opA, opB, M, N, K, A, B, beta, Cin)
    cin = _u16(Cin) if (Cin is not None and beta != 0) else None
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(r.shape, dtype=np.uint16)
    rc = _load(mutation).oracle_gemm_sampled(
        opA, opB, _code(_DTYPES, dtype), M, N, K, float(alpha), _ptr(A, ctypes.c_uint16),
        A.shape[1], _ptr(B, ctypes.c_uint16), B.shape[1], float(beta),
        _ptr(cin, ctypes.c_uint16) if cin is not None else None,
        cin.shape[1] if cin is not None else 0, _ptr(r, ctypes.c_int64), _ptr(c, ctypes.c_int64),
        r.size, _ptr(out, ctypes.c_uint16))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_sampled failed with {rc}")
    return out
