"""CPU oracle for the fp16 / bf16 GEMM and M=1 GEMV: TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never loads it, and it shares no code
with the GPU library: the arithmetic lives in ``sdt_oracle.c`` (plain C, fp64,
ascending-k sums), built by ``make -C oracle``; this module only marshals numpy
arrays into it.

Operand convention (the transposed-B "TN" form C = A @ B_T.T benchmarked in
the FlyDSL pull request "Speed up the RDNA3 GEMM up to 1.85x by choosing the
tile from the shape", Performance section):
  * ``A``: uint16 array of binary16 bit patterns, shape (M, lda), row-major;
    element (m, k) is ``A[m, k]`` for k < K.
  * ``B``: uint16 array, shape (N, ldb); element (k, n) of the math B is
    ``B[n, k]`` (K contiguous, "K-major").
  * result: fp64 array (M, N), unrounded.
Element type: ``dtype="f16"`` (IEEE binary16, the default) or ``"bf16"``
(bfloat16); bit patterns are passed as uint16 either way (a float16 array is
viewed as its bits).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsdt_oracle.so")

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _bits(a) -> np.ndarray:
    """View a float16 or uint16 array as contiguous uint16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected float16/uint16 bit patterns, got {a.dtype}")
    return np.ascontiguousarray(a)


def _p(a, t):
    return a.ctypes.data_as(t)


def _dt(dtype: str) -> int:
    if dtype not in ("f16", "bf16"):
        raise ValueError(f"dtype must be 'f16' or 'bf16', got {dtype!r}")
    return 1 if dtype == "bf16" else 0


class Oracle:
    """The oracle's entry points over one build of ``sdt_oracle.c``.

    The default instance wraps ``oracle/libsdt_oracle.so``; the tests also wrap
    deliberately broken builds to show that the pins catch them."""

    def __init__(self, path: str = _LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(
                f"oracle library {path} is not built; run `make -C {_HERE}`")
        lib = ctypes.CDLL(path)
        lib.sdt_oracle_f16_decode.argtypes = [ctypes.c_uint16]
        lib.sdt_oracle_f16_decode.restype = ctypes.c_double
        lib.sdt_oracle_f16_encode_rne.argtypes = [ctypes.c_double]
        lib.sdt_oracle_f16_encode_rne.restype = ctypes.c_uint16
        lib.sdt_oracle_decode_array.argtypes = [_u16p, _f64p, _i64]
        lib.sdt_oracle_decode_array.restype = None
        lib.sdt_oracle_encode_array.argtypes = [_f64p, _u16p, _i64]
        lib.sdt_oracle_encode_array.restype = None
        lib.sdt_oracle_max_threads.argtypes = []
        lib.sdt_oracle_max_threads.restype = ctypes.c_int
        _c = ctypes.c_int
        lib.sdt_oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        lib.sdt_oracle_bf16_decode.restype = ctypes.c_double
        lib.sdt_oracle_bf16_encode_rne.argtypes = [ctypes.c_double]
        lib.sdt_oracle_bf16_encode_rne.restype = ctypes.c_uint16
        lib.sdt_oracle_bf16_decode_array.argtypes = [_u16p, _f64p, _i64]
        lib.sdt_oracle_bf16_decode_array.restype = None
        lib.sdt_oracle_bf16_encode_array.argtypes = [_f64p, _u16p, _i64]
        lib.sdt_oracle_bf16_encode_array.restype = None
        lib.sdt_oracle_gemm_t.argtypes = [_c, _i64, _i64, _i64, _u16p, _i64, _u16p, _i64,
                                          _f64p, _i64, _c]
        lib.sdt_oracle_gemm_t.restype = _c
        lib.sdt_oracle_gemm_sample_t.argtypes = [_c, _i64, _i64, _i64, _u16p, _i64, _u16p,
                                                 _i64, _i64, _i64p, _i64p, _f64p, _c]
        lib.sdt_oracle_gemm_sample_t.restype = _c
        lib.sdt_oracle_gemv_m1_t.argtypes = [_c, _i64, _i64, _u16p, _u16p, _i64, _f64p, _c]
        lib.sdt_oracle_gemv_m1_t.restype = _c
        lib.sdt_oracle_gemv_kn_t.argtypes = [_c, _i64, _i64, _u16p, _u16p, _i64, _f64p, _c]
        lib.sdt_oracle_gemv_kn_t.restype = _c
        self.path = path
        self._lib = lib

    def f16_decode(self, bits) -> np.ndarray:
        """Exact binary16 -> fp64 decode, elementwise."""
        b = _bits(bits)
        out = np.empty(b.shape, dtype=np.float64)
        self._lib.sdt_oracle_decode_array(_p(b, _u16p), _p(out, _f64p), b.size)
        return out

    def f16_encode_rne(self, x) -> np.ndarray:
        """fp64 -> binary16 bit patterns, round to nearest, ties to even."""
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty(x.shape, dtype=np.uint16)
        self._lib.sdt_oracle_encode_array(_p(x, _f64p), _p(out, _u16p), x.size)
        return out

    def bf16_decode(self, bits) -> np.ndarray:
        """Exact bfloat16 -> fp64 decode of uint16 bit patterns, elementwise."""
        b = _bits(bits)
        out = np.empty(b.shape, dtype=np.float64)
        self._lib.sdt_oracle_bf16_decode_array(_p(b, _u16p), _p(out, _f64p), b.size)
        return out

    def bf16_encode_rne(self, x) -> np.ndarray:
        """fp64 -> bfloat16 bit patterns, round to nearest, ties to even."""
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty(x.shape, dtype=np.uint16)
        self._lib.sdt_oracle_bf16_encode_array(_p(x, _f64p), _p(out, _u16p), x.size)
        return out

    def encode_rne(self, x, dtype: str = "f16") -> np.ndarray:
        return self.bf16_encode_rne(x) if dtype == "bf16" else self.f16_encode_rne(x)

    def max_threads(self) -> int:
        return int(self._lib.sdt_oracle_max_threads())

    def gemm(self, A, B, K: int | None = None, threads: int = 0,
             dtype: str = "f16") -> np.ndarray:
        """C = A.B in fp64 (unrounded); A is (M, lda), B is (N, ldb), K-contiguous."""
        a = _bits(A)
        b = _bits(B)
        if a.ndim != 2 or b.ndim != 2:
            raise ValueError("A and B must be 2-D")
        M, lda = a.shape
        N, ldb = b.shape
        K = lda if K is None else int(K)
        C = np.empty((M, N), dtype=np.float64)
        rc = self._lib.sdt_oracle_gemm_t(_dt(dtype), M, N, K, _p(a, _u16p), lda,
                                         _p(b, _u16p), ldb, _p(C, _f64p), max(N, 1), threads)
        if rc != 0:
            raise ValueError(
                f"oracle gemm rejected M={M} N={N} K={K} lda={lda} ldb={ldb}")
        return C

    def gemm_sample(self, A, B, rows, cols, K: int | None = None,
                    threads: int = 0, dtype: str = "f16") -> np.ndarray:
        """C(rows[i], cols[i]) for each i, by the same definition as :meth:`gemm`."""
        a = _bits(A)
        b = _bits(B)
        M, lda = a.shape
        N, ldb = b.shape
        K = lda if K is None else int(K)
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        c = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
        if r.shape != c.shape:
            raise ValueError("rows and cols must have the same shape")
        out = np.empty(r.shape, dtype=np.float64)
        rc = self._lib.sdt_oracle_gemm_sample_t(_dt(dtype), M, N, K, _p(a, _u16p), lda,
                                                _p(b, _u16p), ldb, r.size, _p(r, _i64p),
                                                _p(c, _i64p), _p(out, _f64p), threads)
        if rc != 0:
            raise ValueError("oracle gemm_sample rejected its arguments")
        return out

    def gemv_m1(self, x, B, K: int | None = None, threads: int = 0,
                dtype: str = "f16") -> np.ndarray:
        """y = x.B in fp64 for the M=1 decode shape; B is (N, ldb), K-contiguous."""
        xv = _bits(x).reshape(-1)
        b = _bits(B)
        N, ldb = b.shape
        K = xv.size if K is None else int(K)
        if xv.size < K:
            raise ValueError("x shorter than K")
        y = np.empty(N, dtype=np.float64)
        rc = self._lib.sdt_oracle_gemv_m1_t(_dt(dtype), N, K, _p(xv, _u16p), _p(b, _u16p),
                                            ldb, _p(y, _f64p), threads)
        if rc != 0:
            raise ValueError("oracle gemv rejected its arguments")
        return y

    def gemv_kn(self, x, B, N: int | None = None, threads: int = 0,
                dtype: str = "f16") -> np.ndarray:
        """y = x.B in fp64 with the weights as K rows of ldb >= N elements
        (B is (K, ldb), the N of one row contiguous)."""
        xv = _bits(x).reshape(-1)
        b = _bits(B)
        K, ldb = b.shape
        N = ldb if N is None else int(N)
        if xv.size < K:
            raise ValueError("x shorter than K")
        y = np.empty(N, dtype=np.float64)
        rc = self._lib.sdt_oracle_gemv_kn_t(_dt(dtype), N, K, _p(xv, _u16p), _p(b, _u16p),
                                            ldb, _p(y, _f64p), threads)
        if rc != 0:
            raise ValueError("oracle gemv_kn rejected its arguments")
        return y


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def f16_decode(bits):
    return default().f16_decode(bits)


def f16_encode_rne(x):
    return default().f16_encode_rne(x)


def max_threads() -> int:
    return default().max_threads()


def bf16_decode(bits):
    return default().bf16_decode(bits)


def bf16_encode_rne(x):
    return default().bf16_encode_rne(x)


def encode_rne(x, dtype="f16"):
    return default().encode_rne(x, dtype)


def gemm(A, B, K=None, threads=0, dtype="f16"):
    return default().gemm(A, B, K, threads, dtype)


def gemm_sample(A, B, rows, cols, K=None, threads=0, dtype="f16"):
    return default().gemm_sample(A, B, rows, cols, K, threads, dtype)


def gemv_m1(x, B, K=None, threads=0, dtype="f16"):
    return default().gemv_m1(x, B, K, threads, dtype)


def gemv_kn(x, B, N=None, threads=0, dtype="f16"):
    return default().gemv_kn(x, B, N, threads, dtype)


def tolerance(c_ref, dtype: str = "f16") -> np.ndarray:
    """Per-element acceptance bound on |C_gpu - C_ref| for K <= 16384, inputs
    uniform in [-1, 1].

    fp16 output: 1e-2 + 2e-3*|C_ref|, the bound this library is held to.  Of
    its relative term, 2^-11 (half an fp16 ulp) pays for rounding the fp32
    result to fp16 and the rest for the fp32 accumulation.
    bf16 output: the same accumulation allowance, with half a bfloat16 ulp
    (2^-8 relative, 8 significant bits) in place of half an fp16 ulp:
    1e-2 + (2e-3 - 2^-11 + 2^-8)*|C_ref| = 1e-2 + 5.42e-3*|C_ref|."""
    rel = 2e-3 if dtype == "f16" else 2e-3 - 2.0 ** -11 + 2.0 ** -8
    if dtype not in ("f16", "bf16"):
        raise ValueError(f"dtype must be 'f16' or 'bf16', got {dtype!r}")
    return 1e-2 + rel * np.abs(np.asarray(c_ref, dtype=np.float64))
