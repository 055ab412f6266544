"""Parity of split-K GEMV (gemv_splitk_*) with the CPU oracle (needs a GPU):
integer inputs bit-exact for every slice count, random inputs within the
bound, the workspace never written past its size, reproducible results."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gemv_inputs as gi
import memory_bound_gemv_f32_amd as lg
from gpu_helpers import (CANARY, GUARD, assert_bit_exact, assert_within_bound, check_guards,
                         guarded_out, run_oracle, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_splitk(case: gi.Case, splits: int = 0, misalign: int = 0):
    """y as float64 (1, M); checks canaries around y and past the end of the
    workspace the library asked for."""
    A, X, bias = upload(case, misalign)
    need = lg.splitk_workspace_size(case.dtype, case.M, case.K, splits)
    n = need // 4
    ws_buf = torch.full((n + GUARD,), CANARY, dtype=torch.float32, device="cuda")
    buf, out = guarded_out((case.M,))
    lg.gemv_splitk(A, X[0], bias, out=out, splits=splits, workspace=ws_buf[:max(n, 1)])
    torch.cuda.synchronize()
    check_guards(buf, case.M)
    tail = ws_buf[n:].cpu().numpy() if n else ws_buf[1:].cpu().numpy()
    assert np.all(tail == np.float32(CANARY)), "write past the workspace"
    return out.cpu().numpy().astype(np.float64)[None, :]


SHAPES = [(1, 64), (7, 1000), (3, 4097), (33, 2048), (5, 129), (2, 100003), (64, 8192)]


@pytest.mark.parametrize("dtype", gi.DTYPES)
@pytest.mark.parametrize("M,K", SHAPES)
def test_integer_bit_exact_every_slice_count(dtype, M, K):
    """Exact-integer regime: every slice count, row pitch and alignment gives
    the exact result (K <= 16384 keeps partial sums exact; larger K uses a
    narrower value range)."""
    hi = 8 if K <= 16384 else 1
    for splits in (0, 1, 2, 3, 7, 64):
        for extra, misalign, bias in ((0, 0, False), (8, 0, True), (0, 1, True), (3, 1, False)):
            case = gi.make_integer(dtype, M, K, seed=M * 131 + K + splits, bias=bias,
                                   lda=K + extra, lo=-hi, hi=hi)
            ref, _ = run_oracle(case)
            got = run_splitk(case, splits, misalign)
            assert_bit_exact(got, ref, f"{dtype} {M}x{K} splits={splits} lda+{extra} "
                                       f"misalign={misalign}")


@pytest.mark.parametrize("dtype", gi.DTYPES)
def test_random_within_bound(dtype):
    for M, K, splits in ((16, 1 << 20, 0), (100, 100000, 0), (1, 1 << 22, 0), (500, 1 << 15, 0),
                         (9, 50000, 13), (1000, 3000, 5)):
        case = gi.make_random(dtype, M, K, seed=M + K, dist="normal", scale=0.02, bias=True)
        ref, absdot = run_oracle(case)
        got = run_splitk(case, splits)
        assert_within_bound(got, ref, absdot, f"{dtype} {M}x{K} splits={splits}")


def test_reproducible_and_close_to_the_single_pass():
    case = gi.make_random("bf16", 32, 1 << 19, seed=5, dist="normal", scale=0.02)
    a = run_splitk(case)
    b = run_splitk(case)
    assert_bit_exact(a, b, "two calls")
    ref, absdot = run_oracle(case)
    A, X, _ = upload(case)
    single = lg.gemv(A, X[0]).cpu().numpy().astype(np.float64)[None, :]
    assert_within_bound(single, ref, absdot, "single pass")
    assert_within_bound(a, ref, absdot, "split")


def test_edge_cases():
    for dtype in gi.DTYPES:
        # K = 0: y = bias whatever the slice count
        case = gi.make_integer(dtype, 5, 0, seed=1, bias=True)
        for splits in (0, 1, 4):
            assert_bit_exact(run_splitk(case, splits), case.bias[None, :].astype(np.float64),
                             "K=0")
        # a NaN planted in one slice of one row reaches that row only
        case = gi.make_integer(dtype, 6, 40000, seed=2, lo=-1, hi=1)
        A = case.A.copy()
        nan = {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}[dtype]
        A[3, 31000] = nan
        planted = gi.Case("nan", dtype, 6, 40000, A, case.X, None, case.lda)
        y = run_splitk(planted, 8)[0]
        assert np.isnan(y[3]) and not np.isnan(np.delete(y, 3)).any()
    # M = 0 is a no-op that needs no workspace
    A = torch.empty((0, 100), dtype=torch.float32, device="cuda")
    x = torch.ones(100, dtype=torch.float32, device="cuda")
    assert lg.gemv_splitk(A, x, splits=4).shape == (0,)


def test_workspace_reused_by_a_smaller_call():
    big = gi.make_integer("f16", 50, 30000, seed=3, lo=-2, hi=2)
    small = gi.make_integer("f16", 3, 9000, seed=4, lo=-2, hi=2)
    ws = torch.empty(lg.splitk_workspace_size("f16", 50, 30000, 20) // 4,
                     dtype=torch.float32, device="cuda")
    for case, splits in ((big, 20), (small, 5), (big, 20)):
        A, X, _ = upload(case)
        y = lg.gemv_splitk(A, X[0], splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert_bit_exact(y.cpu().numpy().astype(np.float64)[None, :], run_oracle(case)[0],
                         f"M={case.M}")


def test_back_to_back_calls_agree():
    """Many calls queued on one stream with one workspace and no wait between
    them give the same bits: the reduce adds each row's partials in an order
    fixed by the slice count alone."""
    case = gi.make_random("f32", 8, 1 << 21, seed=9, dist="normal", scale=0.02, bias=True)
    A, X, bias = upload(case)
    n = lg.splitk_workspace_size("f32", case.M, case.K)
    ws = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    outs = [torch.empty(case.M, dtype=torch.float32, device="cuda") for _ in range(24)]
    for o in outs:
        lg.gemv_splitk(A, X[0], bias, out=o, workspace=ws)
    torch.cuda.synchronize()
    first = outs[0].cpu().numpy()
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(o.cpu().numpy().view(np.uint32), first.view(np.uint32)), f"call {i}"
    ref, absdot = run_oracle(case)
    assert_within_bound(first.astype(np.float64)[None, :], ref, absdot, "f32 8x2^21")


@pytest.mark.parametrize("name", gi.SPLITK_WORKLOADS)
def test_full_size_split_workload(name):
    case = gi.make_workload(name)
    print(f"workload {name}: {case.dtype} M={case.M} K={case.K}", flush=True)
    p = lg.plan_splitk(case.dtype, case.M, case.K)
    assert p["family"] == lg.FAMILY_SPLIT_K
    ref, absdot = run_oracle(case)
    assert_within_bound(run_splitk(case), ref, absdot, name)
