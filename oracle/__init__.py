"""CPU oracle for dense GEMV (TEST INFRASTRUCTURE ONLY).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The product library
(``memory_bound_gemv_f32_amd``) never imports, links or runs it, and this
package imports nothing from the product: the two share no code.

The arithmetic lives in ``gemv_oracle.c`` (plain C, double precision); this
module only compiles it with gcc and marshals numpy arrays through ctypes.
What it computes is the plain definition of GEMV: y[m] is the dot product of
row m of A with x (page "SGEMV CUDA代码学习", section "问题定义: 一行一个点积"),
plus an optional per-row bias that may be absent (page "第 3 课：GEMV 与行级
并行", sections "核心心智模型" item 1 and "3. 正确性边界与指针安全性"), for one
or several right-hand vectors (page "GEMM、GEMV、dtype 与算术强度", section
"可运行 CUDA 实验", the m = 16 small-batch run); the gated SiLU pair and the
weight-only int8 form with a per-row scale (the lqnn.cn NPU MatMul essay,
sections 1.1, 1.2, 4.2, 5.1, 5.2).

Pins: every function here is pinned by tests under ``tests/`` that do not
re-derive it from this code (closed forms, exact integer arithmetic with
``fractions.Fraction``, identity and one-hot matrices, numpy float64 products
and library decoders of fp16/bf16, invariants, planted mistakes).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "gemv_oracle.c"
LIBRARY = HERE / "liboracle_gemv.so"

# dtype codes understood by gemv_oracle.c
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}

# gcc flags: no fast-math and no FMA contraction, so the C source's
# operations are the operations that run.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math"]


def build(source: Path = SOURCE, output: Path = LIBRARY) -> Path:
    """Compile the oracle's C source into a shared library with gcc."""
    tmp = output.with_name(f"{output.name}.tmp{os.getpid()}")
    cmd = ["gcc", *CFLAGS, str(source), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def ensure_built() -> Path:
    """Build the oracle library if it is missing or older than its source."""
    if not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
        build()
    return LIBRARY


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: Path = LIBRARY):
        path = Path(path)
        if path == LIBRARY:
            ensure_built()
        self.path = path
        self._lib = ctypes.CDLL(str(path))
        fn = self._lib.oracle_gemv
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                       ctypes.c_void_p, ctypes.c_void_p]
        self._gemv = fn
        g = self._lib.oracle_gated_silu
        g.restype = ctypes.c_int
        g.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 5
        self._gated = g
        q = self._lib.oracle_gemv_q8
        q.restype = ctypes.c_int
        q.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                      ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        self._q8 = q
        self._lib.oracle_num_threads.restype = ctypes.c_int

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def gemv(self, dtype: str, A: np.ndarray, X: np.ndarray, bias, M: int,
             K: int, lda: int | None = None, nvec: int = 1,
             ldx: int | None = None):
        """Return (Y, ABS), both float64 arrays of shape (nvec, M).

        ``A`` holds at least (M-1)*lda + K stored elements (row-major, row
        stride ``lda``); ``X`` holds ``nvec`` columns of stride ``ldx``
        (default K).  Elements are float32 for ``dtype == "f32"`` and raw
        uint16 bit patterns for ``"f16"`` / ``"bf16"``.  ``bias`` is a float32
        array of length M or None.  Y[j, m] = sum_k A[m,k]·X[j,k] (+ bias[m]),
        ABS[j, m] = sum_k |A[m,k]·X[j,k]|.
        """
        lda = K if lda is None else lda
        ldx = K if ldx is None else ldx
        want = np.float32 if dtype == "f32" else np.uint16
        A = np.ascontiguousarray(A, dtype=want).reshape(-1)
        X = np.ascontiguousarray(X, dtype=want).reshape(-1)
        if M > 0 and K > 0:
            if A.size < (M - 1) * lda + K:
                raise ValueError("A is smaller than its shape implies")
            if X.size < (nvec - 1) * ldx + K:
                raise ValueError("X is smaller than its shape implies")
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32).reshape(-1)
            if bias.size < M:
                raise ValueError("bias is shorter than M")
        Y = np.empty((nvec, max(M, 0)), dtype=np.float64)
        ABS = np.empty_like(Y)
        rc = self._gemv(DTYPE_CODES[dtype],
                        A.ctypes.data if A.size else None, lda,
                        X.ctypes.data if X.size else None, ldx,
                        bias.ctypes.data if bias is not None else None,
                        M, K, nvec, Y.ctypes.data, ABS.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_gemv rejected the arguments (rc={rc})")
        return Y, ABS


    def gated_silu(self, dtype: str, Ag: np.ndarray, Au: np.ndarray, X: np.ndarray,
                   M: int, K: int, lda: int | None = None):
        """h = silu(Ag·x) * (Au·x), with silu(g) = g / (1 + e^-g): the gated
        FFN projection pair.  Returns (H, G, U, ABS_G, ABS_U), each float64
        of shape (M,): G and U are the two products, ABS_* their sums of
        |A·x| (the scale of the GEMV tolerance)."""
        lda = K if lda is None else lda
        want = np.float32 if dtype == "f32" else np.uint16
        Ag = np.ascontiguousarray(Ag, dtype=want).reshape(-1)
        Au = np.ascontiguousarray(Au, dtype=want).reshape(-1)
        X = np.ascontiguousarray(X, dtype=want).reshape(-1)
        if M > 0 and K > 0 and (Ag.size < (M - 1) * lda + K or Au.size < (M - 1) * lda + K
                                or X.size < K):
            raise ValueError("an operand is smaller than its shape implies")
        out = [np.empty(max(M, 0), dtype=np.float64) for _ in range(5)]
        rc = self._gated(DTYPE_CODES[dtype], Ag.ctypes.data if Ag.size else None,
                         Au.ctypes.data if Au.size else None, lda,
                         X.ctypes.data if X.size else None, M, K,
                         *[o.ctypes.data for o in out])
        if rc != 0:
            raise ValueError(f"oracle_gated_silu rejected the arguments (rc={rc})")
        return tuple(out)


    def gemv_q8(self, xdtype: str, Q: np.ndarray, scale, X: np.ndarray, bias, M: int,
                K: int, ldq: int | None = None, nvec: int = 1, ldx: int | None = None):
        """Weight-only int8 GEMV: Y[j, m] = scale[m]·sum_k Q[m,k]·X[j,k]
        (+ bias[m]), ABS[j, m] = |scale[m]|·sum_k |Q[m,k]·X[j,k]|, both
        float64 of shape (nvec, M).  ``Q`` is int8 (row stride ``ldq``),
        ``scale`` float32 (M,), X in the stored encoding of ``xdtype``."""
        ldq = K if ldq is None else ldq
        ldx = K if ldx is None else ldx
        want = np.float32 if xdtype == "f32" else np.uint16
        Q = np.ascontiguousarray(Q, dtype=np.int8).reshape(-1).view(np.uint8)
        X = np.ascontiguousarray(X, dtype=want).reshape(-1)
        scale = np.ascontiguousarray(scale, dtype=np.float32).reshape(-1)
        if M > 0 and K > 0:
            if Q.size < (M - 1) * ldq + K:
                raise ValueError("Q is smaller than its shape implies")
            if X.size < (nvec - 1) * ldx + K:
                raise ValueError("X is smaller than its shape implies")
        if scale.size < M:
            raise ValueError("scale is shorter than M")
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32).reshape(-1)
            if bias.size < M:
                raise ValueError("bias is shorter than M")
        Y = np.empty((nvec, max(M, 0)), dtype=np.float64)
        ABS = np.empty_like(Y)
        rc = self._q8(DTYPE_CODES[xdtype], Q.ctypes.data if Q.size else None, ldq,
                      scale.ctypes.data if scale.size else None,
                      X.ctypes.data if X.size else None, ldx,
                      bias.ctypes.data if bias is not None else None,
                      M, K, nvec, Y.ctypes.data, ABS.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_gemv_q8 rejected the arguments (rc={rc})")
        return Y, ABS


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from this package's own C source."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def gemv(*args, **kwargs):
    return default().gemv(*args, **kwargs)


def gated_silu(*args, **kwargs):
    return default().gated_silu(*args, **kwargs)


def gemv_q8(*args, **kwargs):
    return default().gemv_q8(*args, **kwargs)
