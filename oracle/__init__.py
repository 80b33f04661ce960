"""CPU oracle for the dense GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product path.

The arithmetic lives in ``oracle.c`` (plain C, FP64 accumulation); this module
only builds it with gcc and marshals numpy arrays through ctypes.

What it computes, with citations (page titles and sections):

* "TIRx GEMM on Blackwell", "The short version": D = A @ B.T, FP16 inputs and
  output, FP32 accumulation -> :func:`gemm` with ``layout="nt"``.
* TileFoundry "Choosing schedules and instructions for a backend", section 1
  (GRID HIR): a (M, K) times b (K, N), zero-initialised f32 accumulator, one
  bf16 cast at the end -> :func:`gemm` with ``layout="nn"``.
* The acceptance bound |d_gpu - d| <= ulp_out(|d|) + 2^-11 * sum_k |a*b| ->
  :func:`check`.
* CMU "TIRx" blog, section "Evaluation", "Kernel performance": FP8
  block-scaled matrix multiplication (groups of inputs share a scale) ->
  :func:`gemm_mx`, in the reading stated in ``oracle.c``: E4M3 elements,
  one E8M0 power-of-two scale per 32 consecutive K values of a row, A @ B.T,
  BF16 output.

Parity status: every function here is pinned by CPU tests (exact rational
brute force, invariants, library special cases and the worked values printed
on the pages), the sampled-entry path on both layouts with padded leading
dimensions included; none is "parity unpinned".  The FP8 encodings of gemm_mx
(element and scale formats, group size) are not on the pages: they are the
reading stated in oracle.c, and its pins check that reading.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# tests only: load another build of oracle.c (the planted-mistake tests)
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB")

FMT = {"f16": 0, "bf16": 1}
LAYOUT = {"nt": 0, "nn": 1}

_lib = None


def build() -> str:
    """Compile oracle.c with gcc (no fast-math) into liboracle.so."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    vp = ctypes.c_void_p
    lib.oracle_decode.argtypes = [i32, ctypes.c_uint16]
    lib.oracle_decode.restype = dbl
    lib.oracle_round.argtypes = [i32, dbl]
    lib.oracle_round.restype = ctypes.c_uint16
    lib.oracle_ulp.argtypes = [i32, dbl]
    lib.oracle_ulp.restype = dbl
    lib.oracle_gemm.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, vp, i64]
    lib.oracle_gemm.restype = i32
    lib.oracle_gemm_entries.argtypes = [i32, i32, i64, vp, i64, vp, i64, i64, vp, vp, vp, vp]
    lib.oracle_gemm_entries.restype = None
    lib.oracle_round_array.argtypes = [i32, i64, vp, vp]
    lib.oracle_round_array.restype = None
    lib.oracle_check.argtypes = [i32, i64, vp, vp, vp, vp, vp, vp]
    lib.oracle_check.restype = None
    lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_e4m3.restype = dbl
    lib.oracle_decode_e8m0.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_e8m0.restype = dbl
    lib.oracle_gemm_mx.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, vp, i64]
    lib.oracle_gemm_mx.restype = i32
    lib.oracle_gemm_mx_entries.argtypes = [i64, vp, i64, vp, i64, vp, i64, vp, i64, i64, vp, vp,
                                           vp, vp]
    lib.oracle_gemm_mx_entries.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _bits(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are 16-bit patterns (uint16), got %s" % a.dtype)
    return a


def decode(fmt: str, bits) -> np.ndarray:
    """Exact double value of each 16-bit pattern of format ``fmt``."""
    lib = _load()
    b = _bits(bits)
    out = np.empty(b.shape, dtype=np.float64)
    flat_in, flat_out = b.reshape(-1), out.reshape(-1)
    f = FMT[fmt]
    for t in range(flat_in.size):
        flat_out[t] = lib.oracle_decode(f, int(flat_in[t]))
    return out


def round_to(fmt: str, x) -> np.ndarray:
    """IEEE round-to-nearest-even of doubles to ``fmt``; returns bit patterns."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_round_array(FMT[fmt], x.size, _ptr(x), _ptr(out))
    return out


def ulp(fmt: str, x: float) -> float:
    """Spacing of ``fmt`` at |x| (smallest subnormal at zero)."""
    return _load().oracle_ulp(FMT[fmt], float(x))


def gemm(layout: str, fmt: str, A, B, M=None, N=None, K=None, lda=None, ldb=None):
    """Full product in FP64: returns (d, s), both (M, N) float64.

    ``A`` holds an M x K row-major operand (leading dimension ``lda``); ``B``
    holds N x K (layout "nt") or K x N (layout "nn") with leading dimension
    ``ldb``.  2-D arrays give their own shape and row stride.
    """
    lib = _load()
    A = np.ascontiguousarray(_bits(A))
    B = np.ascontiguousarray(_bits(B))
    if A.ndim == 2:
        M = A.shape[0] if M is None else M
        K = A.shape[1] if K is None else K
        lda = A.shape[1] if lda is None else lda
    if B.ndim == 2:
        if layout == "nt":
            N = B.shape[0] if N is None else N
        else:
            N = B.shape[1] if N is None else N
        ldb = B.shape[1] if ldb is None else ldb
    d = np.empty((M, N), dtype=np.float64)
    s = np.empty((M, N), dtype=np.float64)
    rc = lib.oracle_gemm(LAYOUT[layout], FMT[fmt], M, N, K, _ptr(A), lda, _ptr(B), ldb,
                         _ptr(d), _ptr(s), max(N, 1))
    if rc != 0:
        raise MemoryError("oracle_gemm could not allocate its scratch arrays")
    return d, s


def gemm_entries(layout: str, fmt: str, A, B, K: int, lda: int, ldb: int, rows, cols):
    """Selected elements d[rows[t], cols[t]], s[rows[t], cols[t]] in FP64."""
    lib = _load()
    A = np.ascontiguousarray(_bits(A))
    B = np.ascontiguousarray(_bits(B))
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    d = np.empty(rows.size, dtype=np.float64)
    s = np.empty(rows.size, dtype=np.float64)
    lib.oracle_gemm_entries(LAYOUT[layout], FMT[fmt], K, _ptr(A), lda, _ptr(B), ldb,
                            rows.size, _ptr(rows), _ptr(cols), _ptr(d), _ptr(s))
    return d, s


class CheckResult:
    def __init__(self, n, n_fail, worst_idx, worst_ratio):
        self.n = n
        self.n_fail = n_fail
        self.worst_idx = worst_idx
        self.worst_ratio = worst_ratio

    @property
    def ok(self) -> bool:
        return self.n_fail == 0

    def __repr__(self):
        return ("CheckResult(n=%d, n_fail=%d, worst_idx=%d, worst_ratio=%.4g)"
                % (self.n, self.n_fail, self.worst_idx, self.worst_ratio))


def check(fmt: str, d, s, g_bits) -> CheckResult:
    """Acceptance test |g - d| <= ulp_out(|d|) + 2^-11 * s, elementwise."""
    lib = _load()
    d = np.ascontiguousarray(d, dtype=np.float64).reshape(-1)
    s = np.ascontiguousarray(s, dtype=np.float64).reshape(-1)
    g = np.ascontiguousarray(_bits(g_bits)).reshape(-1)
    if not (d.size == s.size == g.size):
        raise ValueError("check: size mismatch")
    nf = ctypes.c_int64()
    wi = ctypes.c_int64()
    wr = ctypes.c_double()
    lib.oracle_check(FMT[fmt], d.size, _ptr(d), _ptr(s), _ptr(g), ctypes.byref(nf),
                     ctypes.byref(wi), ctypes.byref(wr))
    return CheckResult(d.size, nf.value, wi.value, wr.value)


# ---- FP8 block-scaled (MX) product ------------------------------------------

def _bytes(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError("FP8 operands and E8M0 scales are byte codes (uint8), got %s" % a.dtype)
    return a


def decode_e4m3(codes) -> np.ndarray:
    """Exact double value of each E4M3 byte code (NaN for S.1111.111)."""
    lib = _load()
    c = _bytes(codes)
    return np.array([lib.oracle_decode_e4m3(int(v)) for v in c.reshape(-1)],
                    dtype=np.float64).reshape(c.shape)


def decode_e8m0(codes) -> np.ndarray:
    """2^(e - 127) for each E8M0 byte code (NaN for 255)."""
    lib = _load()
    c = _bytes(codes)
    return np.array([lib.oracle_decode_e8m0(int(v)) for v in c.reshape(-1)],
                    dtype=np.float64).reshape(c.shape)


def gemm_mx(A, SA, B, SB):
    """D = A @ B.T with E4M3 A (M x K), B (N x K) and E8M0 scales SA
    (M x ceil(K/32)), SB (N x ceil(K/32)), all dense 2-D byte arrays.
    Returns (d, s), both (M, N) float64."""
    lib = _load()
    A, SA, B, SB = _bytes(A), _bytes(SA), _bytes(B), _bytes(SB)
    M, K = A.shape
    N = B.shape[0]
    nb = (K + 31) // 32
    if B.shape[1] != K or SA.shape != (M, nb) or SB.shape != (N, nb):
        raise ValueError("gemm_mx: inconsistent shapes")
    d = np.empty((M, N), dtype=np.float64)
    s = np.empty((M, N), dtype=np.float64)
    rc = lib.oracle_gemm_mx(M, N, K, _ptr(A), K, _ptr(SA), nb, _ptr(B), K, _ptr(SB), nb,
                            _ptr(d), _ptr(s), max(N, 1))
    if rc != 0:
        raise MemoryError("oracle_gemm_mx could not allocate its scratch arrays")
    return d, s


def gemm_mx_entries(A, SA, B, SB, rows, cols):
    """Selected elements d[rows[t], cols[t]], s[rows[t], cols[t]] of gemm_mx."""
    lib = _load()
    A, SA, B, SB = _bytes(A), _bytes(SA), _bytes(B), _bytes(SB)
    K = A.shape[1]
    nb = (K + 31) // 32
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    d = np.empty(rows.size, dtype=np.float64)
    s = np.empty(rows.size, dtype=np.float64)
    lib.oracle_gemm_mx_entries(K, _ptr(A), K, _ptr(SA), nb, _ptr(B), K, _ptr(SB), nb,
                               rows.size, _ptr(rows), _ptr(cols), _ptr(d), _ptr(s))
    return d, s
