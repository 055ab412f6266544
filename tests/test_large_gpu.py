"""A matrix of more than 2^31 elements (needs a GPU with several GiB free):
single-vector, batched (matrix cores and vector ALUs) and int8 weights.

The pages' kernels index A with 32-bit int products (row * N + col), which
wrap once M·K reaches 2^31; every offset here is 64-bit.  A (bf16, 4.3 GB)
is built on the device from a closed form with integer values, so every
result is exact in fp32; rows on both sides of the 2^31-element boundary, the
first and last rows and a seeded sample are checked bit for bit against the
oracle, which rebuilds those rows on the host from the same closed form."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import memory_bound_gemv_f32_amd as lg
import oracle

pytestmark = pytest.mark.gpu

M, K = 524_291, 4104          # M·K = 2,151,690,264 > 2^31
BLOCK = 16384


def _row_values(rows: np.ndarray) -> np.ndarray:
    """A[m, k] = ((5m + 3k) mod 17) - 8, an integer in [-8, 8]."""
    k = np.arange(K, dtype=np.int64)
    return ((5 * rows[:, None].astype(np.int64) + 3 * k[None, :]) % 17 - 8).astype(np.float64)


def _x_values() -> np.ndarray:
    return (np.arange(K) % 13 - 6).astype(np.float64)


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    """Integers in [-8, 8] are exact in bfloat16: the top half of the fp32."""
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < 8 << 30:
        pytest.skip("needs 8 GiB of free device memory")


def test_more_than_2_31_elements():
    A = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    k = torch.arange(K, dtype=torch.int32, device="cuda")
    for r0 in range(0, M, BLOCK):
        r1 = min(M, r0 + BLOCK)
        m = torch.arange(r0, r1, dtype=torch.int32, device="cuda")
        A[r0:r1] = ((5 * m[:, None] + 3 * k[None, :]) % 17 - 8).to(torch.bfloat16)
    x = (torch.arange(K, device="cuda") % 13 - 6).to(torch.bfloat16)

    boundary = (1 << 31) // K
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([
        np.arange(0, 64), np.arange(boundary - 64, boundary + 64), np.arange(M - 64, M),
        rng.integers(0, M, size=512)]))
    Ar = _bf16_bits(_row_values(rows))
    xr = _bf16_bits(_x_values())[None, :]
    ref, _ = oracle.gemv("bf16", Ar, xr, None, len(rows), K)
    for family in (lg.FAMILY_AUTO, lg.FAMILY_WAVE_PER_ROW):
        print(f"family {family}: bf16 {M}x{K}", flush=True)
        y = lg.gemv(A, x, family=family)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        np.testing.assert_array_equal(got[rows], ref[0], err_msg=f"family {family}")
        del y

    # three right-hand vectors (x, 2x, -x): the matrix-core and vector-ALU
    # batched kernels
    X = torch.stack([x, 2 * x, -x]).contiguous()
    Xr = np.concatenate([xr, _bf16_bits(2 * _x_values())[None, :], _bf16_bits(-_x_values())[None, :]])
    refb, _ = oracle.gemv("bf16", Ar, Xr, None, len(rows), K, nvec=3)
    for family in (lg.FAMILY_AUTO, lg.FAMILY_BATCHED):
        print(f"batched family {family}: bf16 {M}x{K}, 3 vectors", flush=True)
        Y = lg.gemv_batched(A, X, family=family)
        torch.cuda.synchronize()
        got = Y.cpu().numpy().astype(np.float64)
        np.testing.assert_array_equal(got[:, rows], refb, err_msg=f"batched family {family}")
        del Y
    del A
    torch.cuda.empty_cache()

    # int8 weights of the same closed form, unit scales, fp16 x
    Q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    for r0 in range(0, M, BLOCK):
        r1 = min(M, r0 + BLOCK)
        m = torch.arange(r0, r1, dtype=torch.int32, device="cuda")
        Q[r0:r1] = ((5 * m[:, None] + 3 * k[None, :]) % 17 - 8).to(torch.int8)
    scale = torch.ones(M, dtype=torch.float32, device="cuda")
    xh = (torch.arange(K, device="cuda") % 13 - 6).to(torch.float16)
    xhr = _x_values().astype(np.float16).view(np.uint16)[None, :]
    refq, _ = oracle.gemv_q8("f16", _row_values(rows).astype(np.int8), np.ones(len(rows), np.float32),
                             xhr, None, len(rows), K)
    print(f"int8 {M}x{K}, fp16 x", flush=True)
    y = lg.gemv_q8(Q, scale, xh)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy().astype(np.float64)[rows], refq[0], err_msg="int8")
    del Q, y
    torch.cuda.empty_cache()
