"""gemv_splitk_noalloc: split-K for callers that cannot allocate, with its
partial sums in the library's static device buffer.  Checked through the C
ABI against gemv_splitk_* with a caller's workspace and the same slice
count (the same kernels: the same bits), on calls in a row whose second is
smaller than the first, and against the oracle."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gemv_inputs as gi
import memory_bound_gemv_f32_amd as lg
from gpu_helpers import (assert_bit_exact, assert_within_bound, check_guards, guarded_out,
                         run_oracle, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def with_workspace(case, splits):
    A, X, bias = upload(case)
    y = lg.gemv_splitk(A, X[0], bias, splits=splits)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)[None, :]


def no_alloc(case, splits, expect=lg.GEMV_SUCCESS):
    A, X, bias = upload(case)
    buf, out = guarded_out((case.M,))
    stream = torch.cuda.current_stream().cuda_stream
    rc = lg.gemv_splitk_noalloc(lg.DTYPE_CODES[case.dtype], A.data_ptr(), case.lda, X.data_ptr(),
                                bias.data_ptr() if bias is not None else None, out.data_ptr(),
                                case.M, case.K, splits, stream)
    torch.cuda.synchronize()
    assert rc == expect, (case.dtype, case.M, case.K, splits, rc)
    check_guards(buf, case.M)
    return out.cpu().numpy().astype(np.float64)[None, :]


# (dtype, M, K, splits): the first call of each pair uses most of the
# scratch (M x slices partials), the second is smaller
PAIRS = [(("bf16", 100, 1 << 17, 600), ("bf16", 8, 1 << 16, 0)),
         (("f32", 64, 1 << 18, 0), ("f32", 3, 100003, 7)),
         (("f16", 256, 1 << 16, 250), ("f16", 1, 1 << 20, 0))]


@pytest.mark.parametrize("pair", PAIRS)
def test_matches_the_workspace_entry_point(pair):
    for dtype, M, K, splits in pair:
        need = lg.splitk_workspace_size(dtype, M, K, splits)
        assert 0 < need <= lg.NOALLOC_SCRATCH_BYTES, (dtype, M, K, splits, need)
        case = gi.make_random(dtype, M, K, seed=M + K, bias=M % 2 == 0, dist="normal")
        ref, absdot = run_oracle(case)
        y = no_alloc(case, splits)
        assert_bit_exact(y, with_workspace(case, splits), f"{dtype} {M}x{K} splits={splits}")
        assert_within_bound(y, ref, absdot, f"{dtype} {M}x{K} splits={splits}")


def test_integer_bit_exact_in_a_row():
    for dtype, M, K, splits in (("bf16", 150, 40000, 400), ("f32", 5, 12345, 3), ("f16", 2, 4104, 2)):
        case = gi.make_integer(dtype, M, K, seed=K, bias=True)
        ref, _ = run_oracle(case)
        assert_bit_exact(no_alloc(case, splits), ref, f"{dtype} {M}x{K} splits={splits}")


def test_too_large_for_the_scratch_is_refused():
    case = gi.make_integer("bf16", 1000, 20000, seed=1)
    need = lg.splitk_workspace_size("bf16", 1000, 20000, 100)
    assert need > lg.NOALLOC_SCRATCH_BYTES
    no_alloc(case, 100, expect=lg.GEMV_ERROR_INVALID_VALUE)  # y untouched (guards checked)
    # one slice needs no scratch: the plain single pass runs
    ref, _ = run_oracle(case)
    assert_bit_exact(no_alloc(case, 1), ref, "one slice")
