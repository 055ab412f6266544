"""Pins that tie the CPU oracle to facts outside itself.

Each pin takes an ``oracle.Oracle`` instance and raises ``AssertionError`` if
the oracle disagrees with something the pages or mathematics fix.  None of
them re-types the oracle's formula: expected values come from closed forms,
exact rational arithmetic over library-decoded inputs, numpy's float64
matrix product, structural facts (identity, one-hot, permutations), or from
the pages' own printed shapes.  ``tests/test_oracle.py`` runs them against
the real oracle, and against copies with planted mistakes that must fail.
"""

from __future__ import annotations

import dataclasses
import json
import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import torch

import gemv_inputs as gi

GOLDEN = Path(__file__).resolve().parent / "golden"


# ---------------------------------------------------------------------------
# library decoders (independent of the oracle's hand-written ones)
# ---------------------------------------------------------------------------

def lib_decode(dtype: str, stored: np.ndarray) -> np.ndarray:
    stored = np.asarray(stored)
    if dtype == "f32":
        return stored.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return stored.astype(np.uint16).view(np.float16).astype(np.float64)
    t = torch.from_numpy(stored.astype(np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def _run(oracle, case, **kw):
    return oracle.gemv(case.dtype, case.A, case.X, case.bias, case.M, case.K,
                       lda=case.lda, nvec=case.nvec, **kw)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_worked_example(oracle):
    """Page "第 3 课：GEMV 与行级并行", section "具体演示与数值推演": the M=3,
    K(=N)=1024 walk-through.  With A[m,k] = (m+1)(-1)^k and x[k] = k mod 8,
    every block of 8 consecutive k contributes (0+2+4+6) - (1+3+5+7) = -4
    times (m+1), and there are 1024/8 = 128 blocks, so y[m] = -512 (m+1).
    The sum of |A·x| is (m+1)·128·(0+1+...+7) = 3584 (m+1)."""
    fx = json.loads((GOLDEN / "worked_example_m3_k1024.json").read_text())
    M, K = fx["M"], fx["N"]
    for dtype in gi.DTYPES:
        for with_bias in (False, True):
            case = gi.make_worked_example(dtype, bias=with_bias)
            assert (case.M, case.K) == (M, K)
            Y, S = _run(oracle, case)
            want = [-(K // 8) * 4 * (m + 1) for m in range(M)]
            if with_bias:
                want = [w + b for w, b in zip(want, fx["bias"])]
            assert Y.shape == (1, M)
            assert list(Y[0]) == want, (dtype, with_bias, Y[0], want)
            assert list(S[0]) == [(K // 8) * 28 * (m + 1) for m in range(M)]


def pin_identity(oracle):
    """A = I: y = x (+ bias) exactly, for every encoding."""
    for dtype in gi.DTYPES:
        for with_bias in (False, True):
            case = gi.make_identity(dtype, 67, seed=5, bias=with_bias)
            Y, S = _run(oracle, case)
            want = lib_decode(dtype, case.X[0])
            assert np.array_equal(S[0], np.abs(want))
            if with_bias:
                want = want + case.bias.astype(np.float64)
            assert np.array_equal(Y[0], want), dtype


def pin_one_hot(oracle):
    """One non-zero c_m per row at column pi(m): y[m, j] = c_m · x_j[pi(m)]
    exactly; the NaN padding beyond K (lda > K) must never be read."""
    for dtype in gi.DTYPES:
        for nvec, lda_extra in ((1, 0), (3, 5)):
            case = gi.make_one_hot(dtype, 40, 29, seed=11, nvec=nvec,
                                   lda=29 + lda_extra)
            Y, S = _run(oracle, case)
            X = lib_decode(dtype, case.X)
            for j in range(nvec):
                want = case.coef * X[j, case.cols]
                assert np.array_equal(Y[j], want), (dtype, nvec, j)
                assert np.array_equal(S[j], np.abs(want))


def _exact_reference(case):
    """Exact rational y and sum|A·x| from library-decoded inputs."""
    A = lib_decode(case.dtype, case.A)[:, :case.K] if case.M else np.zeros((0, case.K))
    X = lib_decode(case.dtype, case.X)
    Y = [[None] * case.M for _ in range(case.nvec)]
    S = [[None] * case.M for _ in range(case.nvec)]
    for j in range(case.nvec):
        for m in range(case.M):
            terms = [Fraction(float(A[m, k])) * Fraction(float(X[j, k]))
                     for k in range(case.K)]
            total = sum(terms, Fraction(0))
            if case.bias is not None:
                total += Fraction(float(case.bias[m]))
            Y[j][m] = total
            S[j][m] = sum((abs(t) for t in terms), Fraction(0))
    return Y, S


def pin_brute_force_exact(oracle):
    """Tiny shapes, every encoding, with and without bias, lda > K and
    several vectors: the oracle's double sum must lie within the recursive
    summation bound (K+1)·2^-53·sum|terms| of the exact rational sum, which
    is far tighter than what a float accumulator, a dropped term or a wrong
    index could meet."""
    u = 2.0 ** -53
    seed = 100
    for dtype in gi.DTYPES:
        for M, K in ((1, 0), (1, 1), (2, 3), (3, 5), (4, 8), (3, 17), (2, 33)):
            for with_bias in (False, True):
                for nvec, extra in ((1, 0), (3, 3)):
                    seed += 1
                    case = gi.make_random(dtype, M, K, seed=seed, nvec=nvec,
                                          lda=K + extra, bias=with_bias)
                    Y, S = _run(oracle, case)
                    eY, eS = _exact_reference(case)
                    for j in range(nvec):
                        for m in range(M):
                            bound = (K + 2) * u * float(eS[j][m]) + (
                                u * abs(float(eY[j][m])))
                            err = abs(Fraction(float(Y[j, m])) - eY[j][m])
                            assert float(err) <= bound, (dtype, M, K, j, m)
                            errs = abs(Fraction(float(S[j, m])) - eS[j][m])
                            assert float(errs) <= (K + 2) * u * float(eS[j][m])


def pin_numpy_float64(oracle):
    """numpy's float64 matrix product (a library routine) on random shapes
    with lda > K, several vectors and a bias agrees to 1e-12 of sum|A·x|."""
    for dtype, (M, K, nvec) in (("f32", (131, 1000, 1)), ("f16", (67, 513, 5)),
                                ("bf16", (90, 2049, 3))):
        case = gi.make_random(dtype, M, K, seed=7, nvec=nvec, lda=K + 7,
                              bias=True, dist="normal")
        Y, S = _run(oracle, case)
        A = lib_decode(dtype, case.A)[:, :K]
        X = lib_decode(dtype, case.X)
        want = (A @ X.T).T + case.bias.astype(np.float64)[None, :]
        wantS = (np.abs(A) @ np.abs(X).T).T
        assert Y.shape == (nvec, M)
        assert np.all(np.abs(Y - want) <= 1e-12 * wantS + 1e-300), dtype
        assert np.allclose(S, wantS, rtol=1e-12, atol=0), dtype


def pin_decoders_exhaustive(oracle):
    """Every fp16 and bf16 bit pattern, as a K=1 matrix times x = 1.0, comes
    back as numpy's / torch's decoding of the same bits (NaN where they give
    NaN, infinities and subnormals included)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dtype in ("f16", "bf16"):
        one = gi.quantise(dtype, np.ones((1, 1)))
        Y, _ = oracle.gemv(dtype, bits.reshape(-1, 1), one, None, 1 << 16, 1)
        want = lib_decode(dtype, bits)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(Y[0]), nan), dtype
        # (a -0 element sums to +0: the empty sum starts at +0)
        assert np.array_equal(Y[0][~nan], want[~nan]), dtype
    # binary32: specials, subnormals and random words
    rng = np.random.default_rng(3)
    words = np.concatenate([
        np.array([0, 0x80000000, 1, 0x807FFFFF, 0x00800000, 0x7F7FFFFF,
                  0x7F800000, 0xFF800000, 0x7FC00000, 0x3F800000],
                 dtype=np.uint32),
        rng.integers(0, 1 << 32, size=4000, dtype=np.uint64).astype(np.uint32)])
    f = words.view(np.float32)
    Y, _ = oracle.gemv("f32", f.reshape(-1, 1), np.ones((1, 1), np.float32),
                       None, f.size, 1)
    want = f.astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(Y[0]), nan)
    assert np.array_equal(Y[0][~nan], want[~nan])


def pin_empty_and_degenerate(oracle):
    """K = 0 gives the empty sum: y = bias (or 0) and sum|A·x| = 0.
    M = 0 gives an empty result.  A NaN planted at A[m0, k0] makes y[m0]
    NaN and leaves every other row finite (the row <-> output index)."""
    for dtype in gi.DTYPES:
        case = gi.make_random(dtype, 5, 0, seed=1, bias=True)
        Y, S = oracle.gemv(dtype, np.zeros(0), np.zeros(0), case.bias, 5, 0)
        assert np.array_equal(Y[0], case.bias.astype(np.float64))
        assert np.array_equal(S[0], np.zeros(5))
        Y, _ = oracle.gemv(dtype, np.zeros(0), np.zeros(0), None, 5, 0)
        assert np.array_equal(Y[0], np.zeros(5))
        Y, S = oracle.gemv(dtype, np.zeros(0), np.zeros(0), None, 0, 7)
        assert Y.shape == (1, 0) and S.shape == (1, 0)
        case = gi.make_random(dtype, 9, 21, seed=2, lda=24)
        nan = gi.quantise(dtype, np.array([np.nan]))[0]
        A = case.A.copy()
        A[6, 13] = nan
        Y, _ = oracle.gemv(dtype, A, case.X, None, 9, 21, lda=24)
        assert np.isnan(Y[0, 6])
        assert np.all(np.isfinite(np.delete(Y[0], 6)))


def pin_batched_columns(oracle):
    """Each column of a batched call equals the single-vector call on that
    column, and permuting X's columns permutes Y's columns."""
    for dtype in ("f16", "bf16", "f32"):
        case = gi.make_random(dtype, 23, 70, seed=9, nvec=6, lda=75,
                              bias=True, dist="normal")
        Y, S = _run(oracle, case)
        for j in range(case.nvec):
            y1, s1 = oracle.gemv(dtype, case.A, case.X[j], case.bias, case.M,
                                 case.K, lda=case.lda)
            assert np.array_equal(Y[j], y1[0]) and np.array_equal(S[j], s1[0])
        perm = np.array([4, 0, 5, 2, 1, 3])
        Yp, _ = oracle.gemv(dtype, case.A, case.X[perm], case.bias, case.M,
                            case.K, lda=case.lda, nvec=case.nvec)
        assert np.array_equal(Yp, Y[perm])


def pin_rejects_bad_arguments(oracle):
    """Shapes that describe no problem are refused rather than computed."""
    A = np.zeros(16, np.float32)
    for kw in (dict(M=-1, K=4), dict(M=2, K=-1), dict(M=2, K=4, lda=3),
               dict(M=2, K=4, nvec=0)):
        M, K = kw.pop("M"), kw.pop("K")
        try:
            oracle.gemv("f32", A, A, None, M, K, **kw)
        except ValueError:
            continue
        raise AssertionError(f"accepted M={M} K={K} {kw}")


def pin_worked_example_scaling(oracle):
    """Scaling x by 2 scales y by 2, negating x negates y (exact in every
    encoding for these integer-valued inputs)."""
    for dtype in gi.DTYPES:
        case = gi.make_integer(dtype, 17, 300, seed=4, nvec=2)
        Y, _ = _run(oracle, case)
        X2 = gi.quantise(dtype, 2.0 * lib_decode(dtype, case.X))
        Xn = gi.quantise(dtype, -1.0 * lib_decode(dtype, case.X))
        Y2, _ = oracle.gemv(dtype, case.A, X2, None, case.M, case.K, nvec=2)
        Yn, _ = oracle.gemv(dtype, case.A, Xn, None, case.M, case.K, nvec=2)
        assert np.array_equal(Y2, 2.0 * Y) and np.array_equal(Yn, -Y)


def _torch_silu64(v):
    return torch.nn.functional.silu(torch.from_numpy(np.asarray(v, dtype=np.float64))).numpy()


def pin_gated_silu_against_torch(oracle):
    """h = silu(A_gate·x) * (A_up·x) checked against torch's float64 SiLU
    (a library routine) on exactly known products: with A_gate = A_up = I,
    g = u = x, so h = silu(x)·x; with one-hot rows the products are exact
    and reach |g| up to 64 (both saturated ends of the sigmoid)."""
    for dtype in gi.DTYPES:
        case = gi.make_identity(dtype, 300, seed=3)
        x = lib_decode(dtype, case.X[0]) / 1000.0 * 9.0   # values in [-9, 9]
        X = gi.quantise(dtype, x[None, :])
        xq = lib_decode(dtype, X[0])
        H, G, U, SG, SU = oracle.gated_silu(dtype, case.A, case.A, X, 300, 300)
        want = _torch_silu64(xq) * xq
        assert np.allclose(H, want, rtol=1e-14, atol=1e-300), dtype
        assert np.array_equal(G, xq) and np.array_equal(U, xq)
        oh = gi.make_one_hot(dtype, 200, 50, seed=21)
        oh2 = gi.make_one_hot(dtype, 200, 50, seed=22)
        X = oh.X
        H, G, U, _, _ = oracle.gated_silu(dtype, oh.A, oh2.A, X, 200, 50)
        xv = lib_decode(dtype, X[0])
        g = oh.coef * xv[oh.cols]
        u = oh2.coef * xv[oh2.cols]
        assert np.array_equal(G, g) and np.array_equal(U, u)
        assert np.allclose(H, _torch_silu64(g) * u, rtol=1e-14, atol=1e-300), dtype


def pin_gated_silu_zero_gate(oracle):
    """A zero gate gives silu(0) = 0 for every row whatever the up product;
    a zero up product gives h = 0 whatever the gate."""
    for dtype in gi.DTYPES:
        case = gi.make_random(dtype, 33, 70, seed=8, dist="normal")
        zero = gi.quantise(dtype, np.zeros((33, 70)))
        H, G, U, _, _ = oracle.gated_silu(dtype, zero, case.A, case.X, 33, 70)
        assert np.all(H == 0) and np.all(G == 0) and np.any(U != 0)
        H, G, U, _, _ = oracle.gated_silu(dtype, case.A, zero, case.X, 33, 70)
        assert np.all(H == 0) and np.any(G != 0)


# ---------------------------------------------------------------------------
# weight-only int8 (int8 weights, per-row fp32 scale, float activations)
# ---------------------------------------------------------------------------

def _run_q8(oracle, c, **kw):
    return oracle.gemv_q8(c.xdtype, c.Q, c.scale, c.X, c.bias, c.M, c.K, ldq=c.ldq,
                          nvec=c.nvec, **kw)


def pin_q8_worked_example(oracle):
    """The M=3, K=1024 walk-through with int8 weights (m+1)(-1)^k: the sum
    is -512 (m+1) as for the float case, scaled by 2^-(m+1), so
    y = [-256, -256, -192] (plus the bias); sum|q·x| = 3584 (m+1) scaled
    likewise."""
    for xdtype in gi.DTYPES:
        for with_bias in (False, True):
            c = gi.make_q8_worked_example(xdtype, bias=with_bias)
            Y, S = _run_q8(oracle, c)
            want = [-256.0, -256.0, -192.0]
            if with_bias:
                want = [w + b for w, b in zip(want, (0.5, -0.25, 1.0))]
            assert list(Y[0]) == want, (xdtype, with_bias, Y[0])
            assert list(S[0]) == [3584 * (m + 1) / 2 ** (m + 1) for m in range(3)]


def pin_q8_every_byte(oracle):
    """All 256 int8 bit patterns, one per row at a random column (the rest
    of the row zero), with power-of-two scales: y[m] = scale[m]·q·x[col]
    exactly, q taken from numpy's int8 view of the byte."""
    rng = np.random.default_rng(3)
    M, K = 256, 37
    Q = np.zeros((M, K + 3), dtype=np.int8)
    cols = rng.integers(0, K, size=M)
    Q[np.arange(M), cols] = np.arange(256, dtype=np.uint8).view(np.int8)
    Q[:, K:] = 127                                   # padding, never read
    scale = (2.0 ** rng.integers(-4, 5, size=M)).astype(np.float32)
    for xdtype in gi.DTYPES:
        X = gi.quantise(xdtype, rng.integers(-64, 65, size=(1, K)).astype(np.float64))
        Y, S = oracle.gemv_q8(xdtype, Q, scale, X, None, M, K, ldq=K + 3)
        xv = lib_decode(xdtype, X)[0]
        qv = np.arange(256, dtype=np.uint8).view(np.int8).astype(np.float64)
        want = scale.astype(np.float64) * qv * xv[cols]
        assert np.array_equal(Y[0], want), xdtype
        assert np.array_equal(S[0], np.abs(want)), xdtype


def pin_q8_numpy_float64(oracle):
    """numpy's float64 product of the int8 matrix (as float64) with x, times
    the scale, plus the bias, on random shapes with ldq > K and several
    vectors: agreement to 1e-12 of |scale|·sum|q·x|."""
    for xdtype, (M, K, nvec) in (("f32", (99, 1000, 1)), ("f16", (70, 777, 4)),
                                 ("bf16", (33, 4100, 2))):
        c = gi.make_q8_random(xdtype, M, K, seed=9, nvec=nvec, ldq=K + 5, bias=True)
        Y, S = _run_q8(oracle, c)
        Qf = c.Q[:, :K].astype(np.float64)
        X = lib_decode(xdtype, c.X)
        s = c.scale.astype(np.float64)
        want = (Qf @ X.T).T * s[None, :] + c.bias.astype(np.float64)[None, :]
        wantS = (np.abs(Qf) @ np.abs(X).T).T * np.abs(s)[None, :]
        assert Y.shape == (nvec, M)
        assert np.all(np.abs(Y - want) <= 1e-12 * wantS + 1e-300), xdtype
        assert np.allclose(S, wantS, rtol=1e-12, atol=0), xdtype


def pin_q8_brute_force_exact(oracle):
    """Tiny shapes against exact rational arithmetic: the double result lies
    within (K+3)·2^-53 of |scale|·sum|terms| (+ 2^-53 |y|) of the exact value."""
    u = 2.0 ** -53
    seed = 400
    for xdtype in gi.DTYPES:
        for M, K in ((1, 0), (1, 1), (2, 3), (3, 9), (4, 16), (2, 31)):
            for with_bias, nvec, extra in ((False, 1, 0), (True, 2, 4)):
                seed += 1
                c = gi.make_q8_random(xdtype, M, K, seed=seed, nvec=nvec, ldq=K + extra,
                                      bias=with_bias, q_std=80.0)
                Y, S = _run_q8(oracle, c)
                X = lib_decode(xdtype, c.X)
                for j in range(nvec):
                    for m in range(M):
                        terms = [Fraction(int(c.Q[m, k])) * Fraction(float(X[j, k]))
                                 for k in range(K)]
                        sc = Fraction(float(c.scale[m]))
                        exact = sc * sum(terms, Fraction(0))
                        if with_bias:
                            exact += Fraction(float(c.bias[m]))
                        eS = abs(sc) * sum((abs(t) for t in terms), Fraction(0))
                        bound = (K + 3) * u * float(eS) + u * abs(float(exact))
                        assert float(abs(Fraction(float(Y[j, m])) - exact)) <= bound, (xdtype, M, K)
                        assert float(abs(Fraction(float(S[j, m])) - eS)) <= (K + 3) * u * float(eS)


def pin_q8_scale_and_bias(oracle):
    """Scale 0 gives y = bias exactly; negating the scales negates y exactly
    (no bias); sum|q·x| carries |scale|."""
    for xdtype in gi.DTYPES:
        c = gi.make_q8_random(xdtype, 20, 300, seed=12, bias=True)
        zero = dataclasses.replace(c, scale=np.zeros(20, dtype=np.float32))
        Y, S = _run_q8(oracle, zero)
        assert np.array_equal(Y[0], c.bias.astype(np.float64)) and not S.any()
        nb = dataclasses.replace(c, bias=None)
        neg = dataclasses.replace(nb, scale=-c.scale)
        Yp, Sp = _run_q8(oracle, nb)
        Yn, Sn = _run_q8(oracle, neg)
        assert np.array_equal(Yn, -Yp) and np.array_equal(Sn, Sp)


def pin_q8_rejects_bad_arguments(oracle):
    c = gi.make_q8_random("f16", 4, 8, seed=1)
    for kw in (dict(M=-1), dict(K=-1), dict(ldq=7)):
        args = dict(M=4, K=8, ldq=8)
        args.update(kw)
        try:
            oracle.gemv_q8("f16", c.Q, c.scale, c.X, None, args["M"], args["K"], ldq=args["ldq"])
        except ValueError:
            continue
        raise AssertionError(f"accepted {kw}")


ALL_PINS = [
    pin_worked_example,
    pin_identity,
    pin_one_hot,
    pin_brute_force_exact,
    pin_numpy_float64,
    pin_decoders_exhaustive,
    pin_empty_and_degenerate,
    pin_batched_columns,
    pin_rejects_bad_arguments,
    pin_worked_example_scaling,
    pin_gated_silu_against_torch,
    pin_gated_silu_zero_gate,
    pin_q8_worked_example,
    pin_q8_every_byte,
    pin_q8_numpy_float64,
    pin_q8_brute_force_exact,
    pin_q8_scale_and_bias,
    pin_q8_rejects_bad_arguments,
]


def failing_pins(oracle) -> list[str]:
    """Names of the pins this oracle fails (an exception counts as failing)."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(oracle)
        except Exception:  # noqa: BLE001 - any failure counts
            failed.append(pin.__name__)
    return failed
