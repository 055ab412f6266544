"""Seeded synthetic inputs for GEMV, shared by the tests, the smoke check and
the benchmark.

This module holds no GEMV arithmetic: it only draws random numbers, rounds
them to the stored element types, and lays them out.  Both the HIP path and
the CPU oracle consume the arrays it returns, so they see the same bits.

Element encodings: ``"f32"`` arrays are ``float32``; ``"f16"`` and ``"bf16"``
arrays are ``uint16`` bit patterns.

Workloads (no public dataset or weights are involved; every input is drawn
from a seeded ``numpy.random.default_rng`` in the order A, then x, then bias):

* ``sgemv_1024x128``: fp32, M=1024, K=128, A and x uniform on [-1, 1], no
  bias; the shape timed on page "SGEMV CUDA代码学习" (its opening timing table
  and the benchmark script in section "完整代码"), seed 61.
* ``skinny_k{16,32,128}``: fp32, M=2^20 rows, K in {16, 32, 128}, A, x and
  bias uniform on [-1, 1]; the short-row regime of that page's section
  "Kernel 3: k16" scaled up, seed 62.
* ``decode_f16_4096``: fp16, M=K=4096, A ~ N(0,1)/sqrt(K), x ~ N(0,1), no
  bias; the 4096x4096 fp16 decode (m = 1) run of page "GEMM、GEMV、dtype 与
  算术强度", section "可运行 CUDA 实验", seed 63.
* ``sweep_{q,k,v,o,gate,up,down}``: bf16 decode-layer projections with
  weights ~ N(0, 0.02^2) (0.02 is the standard deviation) and x ~ N(0,1), no
  bias, seeds 640..646.
* ``batched_f16_4096x16``: fp16 W 4096x4096 ~ N(0,1)/sqrt(K), X with 16
  columns (K x 16, column-major) ~ N(0,1), no bias; the m = 16
  small_batch_decode run of the same section, seed 65.
* ``batched_f16_4096x{32,64}``: the same W and X drawn with 32 and 64
  columns, the batch sizes of 16 to 32 and beyond at which page "第 3 课：
  GEMV 与行级并行", section "4. 性能与工程权舍", moves to matrix-core GEMM;
  seeds 70 and 71.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEMENT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


# ---------------------------------------------------------------------------
# rounding float64 draws to the stored encodings (round to nearest, ties even)
# ---------------------------------------------------------------------------

def to_f32(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def to_f16_bits(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(f) -> np.ndarray:
    """Round binary32 values to bfloat16 (ties to even), returning the bits."""
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(f, dtype=np.float32))
    if nan.any():
        sign = ((u >> 16) & 0x8000).astype(np.uint16)
        rounded = np.where(nan, sign | np.uint16(0x7FC0), rounded)
    return rounded.astype(np.uint16)


def to_bf16_bits(v) -> np.ndarray:
    """float64 -> binary32 (ties even) -> bfloat16 (ties even)."""
    return f32_to_bf16_bits(to_f32(v))


def quantise(dtype: str, v) -> np.ndarray:
    if dtype == "f32":
        return to_f32(v)
    if dtype == "f16":
        return to_f16_bits(v)
    if dtype == "bf16":
        return to_bf16_bits(v)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


# ---------------------------------------------------------------------------
# a problem instance
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Case:
    """One GEMV problem: A is (M, lda) stored row-major (columns K..lda-1 are
    padding), X is (nvec, K) (column j of the K x nvec column-major matrix is
    row j here), bias is float32 (M,) or None."""

    name: str
    dtype: str
    M: int
    K: int
    A: np.ndarray
    X: np.ndarray
    bias: np.ndarray | None
    lda: int
    nvec: int = 1
    seed: int | None = None

    def algorithmic_bytes(self) -> int:
        return workload_bytes(self.dtype, self.M, self.K, self.nvec,
                              self.bias is not None)


def workload_bytes(dtype: str, M: int, K: int, nvec: int = 1,
                   has_bias: bool = False) -> int:
    """Minimum HBM bytes of one call: A read once, every x column read once,
    y written once as fp32, bias read once if present."""
    s = ELEMENT_BYTES[dtype]
    return M * K * s + nvec * K * s + 4 * M * nvec + (4 * M if has_bias else 0)


def workload_flops(M: int, K: int, nvec: int = 1, has_bias: bool = False) -> int:
    return 2 * M * K * nvec + (M * nvec if has_bias else 0)


def _pad(A: np.ndarray, lda: int, fill) -> np.ndarray:
    M, K = A.shape
    if lda == K:
        return np.ascontiguousarray(A)
    out = np.full((M, lda), fill, dtype=A.dtype)
    out[:, :K] = A
    return out


def _padding_value(dtype: str):
    """A quiet NaN in the stored encoding: padding that must never be read."""
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "f16":
        return np.uint16(0x7E00)
    return np.uint16(0x7FC0)


def make_random(dtype: str, M: int, K: int, *, seed: int, nvec: int = 1,
                lda: int | None = None, bias: bool = False,
                dist: str = "uniform", scale: float = 1.0,
                name: str | None = None) -> Case:
    """Random case: ``dist`` is "uniform" (on [-scale, scale]) or "normal"
    (standard deviation ``scale`` for A; x and bias are drawn like A but with
    scale 1 for "normal")."""
    rng = np.random.default_rng(seed)
    lda = K if lda is None else lda
    if dist == "uniform":
        a = rng.uniform(-scale, scale, size=(M, K))
        x = rng.uniform(-1.0, 1.0, size=(nvec, K))
        b = rng.uniform(-1.0, 1.0, size=M) if bias else None
    elif dist == "normal":
        a = rng.standard_normal(size=(M, K)) * scale
        x = rng.standard_normal(size=(nvec, K))
        b = rng.standard_normal(size=M) if bias else None
    else:
        raise ValueError(dist)
    A = _pad(quantise(dtype, a), lda, _padding_value(dtype))
    X = np.ascontiguousarray(quantise(dtype, x))
    return Case(name or f"rand_{dtype}_{M}x{K}", dtype, M, K, A, X,
                None if b is None else to_f32(b), lda, nvec, seed)


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

SWEEP_SHAPES = {           # name: (M, K)
    "q": (4096, 4096),
    "k": (1024, 4096),
    "v": (1024, 4096),
    "o": (4096, 4096),
    "gate": (14336, 4096),
    "up": (14336, 4096),
    "down": (4096, 14336),
}

WORKLOADS = {
    # name: (dtype, M, K, nvec, bias, dist, scale rule, seed)
    "sgemv_1024x128": ("f32", 1024, 128, 1, False, "uniform", None, 61),
    "skinny_k16": ("f32", 1 << 20, 16, 1, True, "uniform", None, 62),
    "skinny_k32": ("f32", 1 << 20, 32, 1, True, "uniform", None, 62),
    "skinny_k128": ("f32", 1 << 20, 128, 1, True, "uniform", None, 62),
    "decode_f16_4096": ("f16", 4096, 4096, 1, False, "normal", "1/sqrtK", 63),
    "batched_f16_4096x16": ("f16", 4096, 4096, 16, False, "normal", "1/sqrtK", 65),
    "batched_f16_4096x32": ("f16", 4096, 4096, 32, False, "normal", "1/sqrtK", 70),
    "batched_f16_4096x64": ("f16", 4096, 4096, 64, False, "normal", "1/sqrtK", 71),
}
for _i, (_n, (_m, _k)) in enumerate(SWEEP_SHAPES.items()):
    WORKLOADS[f"sweep_{_n}"] = ("bf16", _m, _k, 1, False, "normal", 0.02, 640 + _i)
# few, long rows (the split-K case): the small-M example of the SGEMV page
# (M = 8) with 2^21-element fp32 rows, and 64 bf16 rows of 2^18 elements
WORKLOADS["splitk_f32_8x2M"] = ("f32", 8, 1 << 21, 1, False, "uniform", None, 66)
WORKLOADS["splitk_bf16_64x256k"] = ("bf16", 64, 1 << 18, 1, False, "normal", 0.02, 67)
SPLITK_WORKLOADS = ("splitk_f32_8x2M", "splitk_bf16_64x256k")


def workload_shape(name: str):
    dtype, M, K, nvec, bias, _, _, _ = WORKLOADS[name]
    return dtype, M, K, nvec, bias


def make_workload(name: str, lda: int | None = None) -> Case:
    dtype, M, K, nvec, bias, dist, rule, seed = WORKLOADS[name]
    if rule is None:
        scale = 1.0
    elif rule == "1/sqrtK":
        scale = 1.0 / math.sqrt(K)
    else:
        scale = float(rule)
    return make_random(dtype, M, K, seed=seed, nvec=nvec, lda=lda, bias=bias,
                       dist=dist, scale=scale, name=name)


# ---------------------------------------------------------------------------
# structured inputs whose products are known in closed form
# ---------------------------------------------------------------------------

def make_integer(dtype: str, M: int, K: int, *, seed: int, nvec: int = 1,
                 lda: int | None = None, bias: bool = False,
                 lo: int = -8, hi: int = 8) -> Case:
    """Integer-valued A, x (and bias) in [lo, hi]: exact in every encoding, and
    for K <= 16384 every partial sum stays below 2^24, so any fp32 summation
    order gives the exact result."""
    rng = np.random.default_rng(seed)
    lda = K if lda is None else lda
    a = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float64)
    x = rng.integers(lo, hi + 1, size=(nvec, K)).astype(np.float64)
    b = rng.integers(lo, hi + 1, size=M).astype(np.float64) if bias else None
    A = _pad(quantise(dtype, a), lda, _padding_value(dtype))
    return Case(f"int_{dtype}_{M}x{K}", dtype, M, K, A,
                np.ascontiguousarray(quantise(dtype, x)),
                None if b is None else to_f32(b), lda, nvec, seed)


def make_worked_example(dtype: str, bias: bool = False) -> Case:
    """M=3, K=1024 with A[m,k] = (m+1)·(-1)^k and x[k] = k mod 8, and bias
    [0.5, -0.25, 1] when requested: the shape walked through on page "第 3 课：
    GEMV 与行级并行", section "具体演示与数值推演" (the page prints no values;
    these entries are chosen so every value is exact in every encoding)."""
    M, K = 3, 1024
    k = np.arange(K)
    a = np.array([(m + 1) * np.where(k % 2 == 0, 1.0, -1.0) for m in range(M)])
    x = (k % 8).astype(np.float64)[None, :]
    b = np.array([0.5, -0.25, 1.0]) if bias else None
    return Case(f"worked_{dtype}", dtype, M, K, quantise(dtype, a),
                quantise(dtype, x), None if b is None else to_f32(b), K)


def make_identity(dtype: str, n: int, *, seed: int, bias: bool = False) -> Case:
    """A = I (n x n), x random integer-valued in [-1000, 1000] (exact in fp16
    and fp32; bf16 rounds x once at quantisation, which is the stored x)."""
    rng = np.random.default_rng(seed)
    a = np.eye(n)
    x = rng.integers(-1000, 1001, size=(1, n)).astype(np.float64)
    b = rng.integers(-50, 51, size=n).astype(np.float64) if bias else None
    return Case(f"identity_{dtype}_{n}", dtype, n, n, quantise(dtype, a),
                quantise(dtype, x), None if b is None else to_f32(b), n, 1, seed)


def make_one_hot(dtype: str, M: int, K: int, *, seed: int, nvec: int = 1,
                 lda: int | None = None) -> Case:
    """Row m of A has one non-zero entry c_m (a power of two in
    [2^-3, 2^3], random sign) at column pi(m), a random column; x is random
    integer-valued.  Then y[m] = c_m · x[pi(m)] exactly."""
    rng = np.random.default_rng(seed)
    lda = K if lda is None else lda
    cols = rng.integers(0, K, size=M)
    coef = (2.0 ** rng.integers(-3, 4, size=M)) * rng.choice([-1.0, 1.0], size=M)
    a = np.zeros((M, K))
    a[np.arange(M), cols] = coef
    x = rng.integers(-64, 65, size=(nvec, K)).astype(np.float64)
    A = _pad(quantise(dtype, a), lda, _padding_value(dtype))
    case = Case(f"onehot_{dtype}_{M}x{K}", dtype, M, K, A,
                np.ascontiguousarray(quantise(dtype, x)), None, lda, nvec, seed)
    case.cols = cols          # the column of each row's non-zero entry
    case.coef = coef          # and its value
    return case


# ---------------------------------------------------------------------------
# fused decode workloads: the sweep's matrices, one shared x
# ---------------------------------------------------------------------------

def make_fused_qkv() -> list[Case]:
    """The q, k and v projections of the decode-layer sweep as one problem:
    their matrices (seeds 640..642) and the q workload's x for all three."""
    parts = [make_workload(f"sweep_{n}") for n in ("q", "k", "v")]
    for p in parts[1:]:
        p.X = parts[0].X
    return parts


def make_fused_gate_up() -> tuple[Case, Case]:
    """The gate and up projections of the sweep (seeds 644, 645), sharing the
    gate workload's x."""
    gate, up = make_workload("sweep_gate"), make_workload("sweep_up")
    up.X = gate.X
    return gate, up


# ---------------------------------------------------------------------------
# weight-only int8 problems: int8 weights, one fp32 scale per row, float x
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Q8Case:
    """Q is (M, ldq) int8 row-major (columns K..ldq-1 are padding, filled
    with -128 so that a stray read changes a result), scale is float32 (M,),
    X is (nvec, K) in the stored encoding of ``xdtype``, bias float32 (M,)
    or None."""

    name: str
    xdtype: str
    M: int
    K: int
    Q: np.ndarray
    scale: np.ndarray
    X: np.ndarray
    bias: np.ndarray | None
    ldq: int
    nvec: int = 1
    seed: int | None = None

    def algorithmic_bytes(self) -> int:
        return q8_bytes(self.xdtype, self.M, self.K, self.nvec, self.bias is not None)


def q8_bytes(xdtype: str, M: int, K: int, nvec: int = 1, has_bias: bool = False) -> int:
    """Q once (1 byte per weight), the scales, x once, y once (fp32)."""
    s = ELEMENT_BYTES[xdtype]
    return M * K + 4 * M + nvec * K * s + 4 * M * nvec + (4 * M if has_bias else 0)


def _pad_q(q: np.ndarray, ldq: int) -> np.ndarray:
    M, K = q.shape
    out = np.full((M, ldq), -128, dtype=np.int8)
    out[:, :K] = q
    return out


def make_q8_random(xdtype: str, M: int, K: int, *, seed: int, nvec: int = 1,
                   ldq: int | None = None, bias: bool = False, q_std: float = 32.0,
                   w_std: float = 0.02, name: str | None = None) -> Q8Case:
    """Bell-shaped int8 weights (normal with standard deviation ``q_std``,
    rounded and clipped to [-127, 127], as weights of standard deviation
    ``w_std`` look after a per-row absmax scaling), per-row scales near
    4·w_std/127, x ~ N(0, 1) in ``xdtype``."""
    rng = np.random.default_rng(seed)
    ldq = K if ldq is None else ldq
    q = np.clip(np.rint(rng.standard_normal((M, K)) * q_std), -127, 127).astype(np.int8)
    scale = to_f32(4.0 * w_std / 127.0 * rng.uniform(0.8, 1.2, size=M))
    x = rng.standard_normal((nvec, K))
    b = rng.standard_normal(M) if bias else None
    return Q8Case(name or f"q8_{xdtype}_{M}x{K}", xdtype, M, K, _pad_q(q, ldq), scale,
                  np.ascontiguousarray(quantise(xdtype, x)), None if b is None else to_f32(b),
                  ldq, nvec, seed)


def make_q8_integer(xdtype: str, M: int, K: int, *, seed: int, nvec: int = 1,
                    ldq: int | None = None, bias: bool = False, lo: int = -8,
                    hi: int = 8) -> Q8Case:
    """Every int8 value in Q, integer x in [lo, hi], power-of-two scales
    2^-e (e in 0..6) and integer bias: for K·128·max(|lo|, |hi|) < 2^24
    every partial sum is exact in fp32, and so is the scaled result."""
    rng = np.random.default_rng(seed)
    ldq = K if ldq is None else ldq
    q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    scale = to_f32(2.0 ** -rng.integers(0, 7, size=M))
    x = rng.integers(lo, hi + 1, size=(nvec, K)).astype(np.float64)
    b = rng.integers(lo, hi + 1, size=M).astype(np.float64) if bias else None
    return Q8Case(f"q8int_{xdtype}_{M}x{K}", xdtype, M, K, _pad_q(q, ldq), scale,
                  np.ascontiguousarray(quantise(xdtype, x)), None if b is None else to_f32(b),
                  ldq, nvec, seed)


def make_q8_worked_example(xdtype: str, bias: bool = False) -> Q8Case:
    """The M=3, K=1024 walk-through with int8 weights Q[m,k] = (m+1)(-1)^k,
    x[k] = k mod 8 and scales 2^-(m+1)."""
    M, K = 3, 1024
    k = np.arange(K)
    q = np.array([(m + 1) * (-1.0) ** k for m in range(M)]).astype(np.int8)
    x = (k % 8).astype(np.float64)[None, :]
    scale = to_f32([2.0 ** -(m + 1) for m in range(M)])
    b = to_f32([0.5, -0.25, 1.0]) if bias else None
    return Q8Case(f"q8_worked_{xdtype}", xdtype, M, K, _pad_q(q, K), scale,
                  np.ascontiguousarray(quantise(xdtype, x)), b, K)


# the int8 forms of the decode sweep's q/o and gate/up shapes: int8 weights,
# fp16 (q/o) or bf16 (gate/up) activations
Q8_WORKLOADS = {
    # name: (xdtype, M, K, seed)
    "q8_f16_4096": ("f16", 4096, 4096, 68),
    "q8_bf16_14336x4096": ("bf16", 14336, 4096, 69),
    "q8_f16_4096x11008": ("f16", 4096, 11008, 70),
}


def make_q8_workload(name: str) -> Q8Case:
    xdtype, M, K, seed = Q8_WORKLOADS[name]
    return make_q8_random(xdtype, M, K, seed=seed, name=name)


def fused_qkv_bytes() -> int:
    """A of q, k, v once, x once, y of all three once."""
    M = sum(SWEEP_SHAPES[n][0] for n in ("q", "k", "v"))
    K = SWEEP_SHAPES["q"][1]
    return M * K * 2 + K * 2 + 4 * M


def fused_gate_up_bytes() -> int:
    """Both matrices once, x once, h once (fp32)."""
    M, K = SWEEP_SHAPES["gate"]
    return 2 * M * K * 2 + K * 2 + 4 * M
