"""Parity of the fused decode entry points with the CPU oracle (needs a GPU):
gemv_multi_* (several matrices sharing x in one launch) and
gemv_gate_up_silu_* (h = silu(A_gate·x) · (A_up·x))."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gemv_inputs as gi
import memory_bound_gemv_f32_amd as lg
import oracle
from gpu_helpers import (assert_bit_exact, assert_within_bound,
                         check_guards, guarded_out, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_multi(cases, misalign=0):
    """cases share K, dtype and (the first case's) x; returns per-case
    float64 outputs, checking canaries around each."""
    dt = cases[0].dtype
    x = to_device(dt, cases[0].X[0], misalign)
    As, biases, bufs, outs = [], [], [], []
    for c in cases:
        A_full = to_device(dt, c.A.reshape(c.M, c.lda), misalign)
        As.append(A_full[:, :c.K])
        biases.append(None if c.bias is None else torch.from_numpy(c.bias).cuda())
        buf, out = guarded_out((c.M,))
        bufs.append(buf)
        outs.append(out)
    lg.gemv_multi(As, x, biases, outs)
    torch.cuda.synchronize()
    res = []
    for c, buf, out in zip(cases, bufs, outs):
        check_guards(buf, c.M)
        res.append(out.cpu().numpy().astype(np.float64))
    return res


def oracle_multi(cases):
    out = []
    for c in cases:
        Y, S = oracle.gemv(c.dtype, c.A, cases[0].X, c.bias, c.M, c.K, lda=c.lda)
        out.append((Y[0], S[0]))
    return out


@pytest.mark.parametrize("dtype", gi.DTYPES)
@pytest.mark.parametrize("Ms,K", [([4096, 1024, 1024], 4096), ([5, 0, 300, 1, 77], 1000),
                                  ([1000, 1000], 16), ([3] * 8, 129), ([64], 14336),
                                  ([2000, 17, 9000], 100)])
def test_multi_integer_bit_exact(dtype, Ms, K):
    cases = [gi.make_integer(dtype, M, K, seed=M + 3 * i, bias=i % 2 == 0, lda=K + (i % 3))
             for i, M in enumerate(Ms)]
    got = run_multi(cases)
    for c, g, (ref, _) in zip(cases, got, oracle_multi(cases)):
        assert_bit_exact(g[None, :], ref[None, :], f"{dtype} segment M={c.M}")


@pytest.mark.parametrize("dtype", gi.DTYPES)
@pytest.mark.parametrize("Ms,K", [([4096, 1024, 1024], 4096), ([5, 0, 300], 1000),
                                  ([1000, 1000], 16), ([64], 14336), ([0, 17, 9000], 100),
                                  ([3000, 1, 6000], 600), ([200, 56], 5000)])
@pytest.mark.parametrize("bias", ["none", "middle", "all"])
def test_multi_three_segments_one_pitch(dtype, Ms, K, bias):
    """At most three matrices of one row pitch run the kernels that take the
    segment table as scalar arguments: every family, empty segments, a bias
    on some segments only; bit-exact."""
    lda = K + (3 if K % 2 else 0)
    def has_bias(i):
        return bias == "all" or (bias == "middle" and i == 1)
    cases = [gi.make_integer(dtype, M, K, seed=M + 5 * i, bias=has_bias(i), lda=lda)
             for i, M in enumerate(Ms)]
    got = run_multi(cases)
    for c, g, (ref, _) in zip(cases, got, oracle_multi(cases)):
        assert_bit_exact(g[None, :], ref[None, :], f"{dtype} segment M={c.M} bias={bias}")


@pytest.mark.parametrize("dtype", gi.DTYPES)
@pytest.mark.parametrize("misalign", [0, 1])
def test_multi_random_within_bound(dtype, misalign):
    K = 2048
    pad = 8 if dtype != "f32" else 4
    cases = [gi.make_random(dtype, M, K, seed=50 + M, bias=True, dist="normal",
                            lda=K + pad * (i % 2)) for i, M in enumerate([1024, 333, 4096, 1])]
    got = run_multi(cases, misalign)
    for c, g, (ref, s) in zip(cases, got, oracle_multi(cases)):
        assert_within_bound(g[None, :], ref[None, :], s[None, :], f"{dtype} M={c.M}")


def test_multi_one_hot_boundaries():
    """One-hot rows in each segment: any row-to-segment mix-up at a segment
    boundary changes an output exactly."""
    for dtype in gi.DTYPES:
        cases = [gi.make_one_hot(dtype, M, 300, seed=M) for M in (7, 64, 1, 129, 4)]
        got = run_multi(cases)
        for c, g, (ref, _) in zip(cases, got, oracle_multi(cases)):
            assert_bit_exact(g[None, :], ref[None, :], f"{dtype} one-hot M={c.M}")


def test_multi_matches_the_decode_projections():
    q, k, v = gi.make_fused_qkv()
    got = run_multi([q, k, v])
    for c, g, (ref, s) in zip((q, k, v), got, oracle_multi([q, k, v])):
        assert_within_bound(g[None, :], ref[None, :], s[None, :], f"fused {c.name}")


# ---------------------------------------------------------------------------
# gated pair
# ---------------------------------------------------------------------------

def gated_bound(G, U, SG, SU, H):
    """From the GEMV bound on g and u: silu has slope at most about 1.1."""
    tg = 1e-5 * SG + 1e-6
    tu = 1e-5 * SU + 1e-6
    with np.errstate(over="ignore"):
        silu_g = G / (1.0 + np.exp(-G))
    return 1.1 * tg * (np.abs(U) + tu) + np.abs(silu_g) * tu + 1e-6 * np.abs(H) + 1e-6


def run_gated(gate: gi.Case, up: gi.Case, misalign=0):
    dt = gate.dtype
    Ag = to_device(dt, gate.A.reshape(gate.M, gate.lda), misalign)[:, :gate.K]
    Au = to_device(dt, up.A.reshape(up.M, up.lda), misalign)[:, :up.K]
    x = to_device(dt, gate.X[0], misalign)
    buf, out = guarded_out((gate.M,))
    lg.gemv_gate_up_silu(Ag, Au, x, out)
    torch.cuda.synchronize()
    check_guards(buf, gate.M)
    return out.cpu().numpy().astype(np.float64)


def check_gated(gate, up, misalign=0, what=""):
    h = run_gated(gate, up, misalign)
    H, G, U, SG, SU = oracle.gated_silu(gate.dtype, gate.A, up.A, gate.X[0], gate.M, gate.K,
                                        lda=gate.lda)
    err = np.abs(h - H)
    bound = gated_bound(G, U, SG, SU, H)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {bad.sum()} rows outside the bound; first "
                           f"{np.argwhere(bad)[:3].ravel()} got {h[bad][:3]} want {H[bad][:3]}")


@pytest.mark.parametrize("dtype", gi.DTYPES)
@pytest.mark.parametrize("M,K", [(1, 64), (100, 4096), (1000, 1000), (4096, 4096),
                                 (9000, 512), (64, 14336), (333, 17), (14336, 4096)])
def test_gated_within_bound(dtype, M, K):
    for misalign, extra in ((0, 0), (0, 8), (1, 0)):
        gate = gi.make_random(dtype, M, K, seed=M + K, dist="normal", scale=0.05, lda=K + extra)
        up = gi.make_random(dtype, M, K, seed=M + K + 1, dist="normal", scale=0.05, lda=K + extra)
        check_gated(gate, up, misalign, f"{dtype} {M}x{K} lda+{extra} misalign {misalign}")


def test_gated_exact_cases():
    """A zero gate gives exactly 0 (silu(0) = 0), as does K = 0; a zero up
    matrix gives exactly 0 whatever the gate."""
    for dtype in gi.DTYPES:
        up = gi.make_random(dtype, 500, 300, seed=1, dist="normal")
        zero = gi.Case("zero", dtype, 500, 300, gi.quantise(dtype, np.zeros((500, 300))),
                       up.X, None, 300)
        assert np.all(run_gated(zero, up) == 0)
        assert np.all(run_gated(up, zero) == 0)
        empty = gi.Case("empty", dtype, 50, 0, gi.quantise(dtype, np.zeros((50, 0))),
                        gi.quantise(dtype, np.zeros((1, 0))), None, 0)
        assert np.all(run_gated(empty, empty) == 0)


def test_gated_decode_gate_up():
    gate, up = gi.make_fused_gate_up()
    check_gated(gate, up, what="decode gate/up 14336x4096")
