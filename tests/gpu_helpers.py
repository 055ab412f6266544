"""Helpers for the GPU parity tests: upload seeded inputs, call libgemv through
its C ABI, and compare with the CPU oracle."""

from __future__ import annotations

import numpy as np
import torch

import gemv_inputs as gi
import oracle

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM = {"f32": 4, "f16": 2, "bf16": 2}
CANARY = 12345.678
GUARD = 64


def to_device(dtype: str, arr: np.ndarray, misalign: int = 0):
    """Copy a stored-encoding array to the GPU, optionally starting
    ``misalign`` elements into a larger allocation (so the pointer is only
    element-aligned).  Returns a tensor of the matching torch dtype with the
    array's shape."""
    flat = np.ascontiguousarray(arr).reshape(-1)
    if dtype == "f32":
        host = torch.from_numpy(flat.astype(np.float32))
    else:
        host = torch.from_numpy(flat.astype(np.uint16).view(np.int16)).view(TORCH_DTYPE[dtype])
    buf = torch.empty(flat.size + misalign + 8, dtype=TORCH_DTYPE[dtype], device="cuda")
    dev = buf[misalign:misalign + flat.size]
    dev.copy_(host)
    return dev.view(arr.shape)


def upload(case: gi.Case, misalign: int = 0):
    """Device A (as an (M, K) view with row stride lda), X and bias."""
    A_full = to_device(case.dtype, case.A.reshape(case.M, case.lda), misalign)
    A = A_full[:, :case.K]
    X = to_device(case.dtype, case.X.reshape(case.nvec, case.K), misalign)
    bias = None
    if case.bias is not None:
        bias = torch.from_numpy(case.bias.astype(np.float32)).cuda()
    return A, X, bias


def guarded_out(shape):
    """An output tensor with canary words before and after it."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.float32, device="cuda")
    return buf, buf[GUARD:GUARD + n].view(shape)


def check_guards(buf, n):
    host = buf.cpu().numpy()
    assert np.all(host[:GUARD] == np.float32(CANARY)), "write before y[0]"
    assert np.all(host[GUARD + n:] == np.float32(CANARY)), "write after y[M-1]"


def run_gpu(case: gi.Case, family: int, *, misalign: int = 0, batched: bool = False):
    """Run libgemv on ``case``; returns Y as float64 (nvec, M) and checks the
    canary words around the output."""
    import memory_bound_gemv_f32_amd as lg
    A, X, bias = upload(case, misalign)
    buf, out = guarded_out((case.nvec, case.M))
    if batched or case.nvec > 1:
        lg.gemv_batched(A, X, bias, out=out, family=family)
    else:
        lg.gemv(A, X[0], bias, out=out[0], family=family)
    torch.cuda.synchronize()
    check_guards(buf, case.nvec * case.M)
    return out.cpu().numpy().astype(np.float64)


def run_oracle(case: gi.Case):
    return oracle.gemv(case.dtype, case.A, case.X, case.bias, case.M, case.K,
                       lda=case.lda, nvec=case.nvec)


def assert_within_bound(y, ref, absdot, what=""):
    """|y - ref| <= 1e-5 * sum_k |A[m,k] x[k]| + 1e-6 for every output."""
    err = np.abs(y - ref)
    bound = 1e-5 * absdot + 1e-6
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: got {y[tuple(i)]!r} want {ref[tuple(i)]!r} "
                           f"bound {bound[tuple(i)]:.3g}" for i in idx)
        raise AssertionError(f"{what}: {bad.sum()} outputs outside the bound; {detail}")


def assert_bit_exact(y, ref, what=""):
    if not np.array_equal(y, ref):
        idx = np.argwhere(y != ref)[:5]
        detail = ", ".join(f"{tuple(i)}: got {y[tuple(i)]!r} want {ref[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: not bit-exact; {detail}")
