"""Brute force over tiny shapes on the GPU: every accepted kernel family
(the automatic choice and each forced one), every element type, rows M in
{1, 2, 3, 5, 9}, lengths K = 0..130 and the bands around 256, 512, 1024 and
4096, row pitches K, K+1 and K+8 (padding filled with NaN, so a read past K
shows), element-aligned pointers, with and without a bias; then the batched
entry points with 2-64 vectors on the lengths the matrix cores take.  All
data are small integers, so every result is exact in fp32 whatever the
summation order and must equal the oracle bit for bit; guard words around
every result must be untouched.  (Page "第 3 课：GEMV 与行级并行", sections
"评分与通过规则" and "3. 正确性边界与指针安全性": normal and boundary inputs,
no access past the data.)

All cases of one element type share one input upload, one output buffer and
one synchronisation, so the sweep takes seconds.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gemv_inputs as gi
import memory_bound_gemv_f32_amd as lg
import oracle

pytestmark = pytest.mark.gpu

M_VALUES = (1, 2, 3, 5, 9)
K_VALUES = list(range(0, 131)) + [255, 256, 257, 511, 512, 513, 1023, 1024, 1025,
                                  4095, 4096, 4097]
K_BATCHED = [k for k in K_VALUES if k % 8 == 0]
NVECS = (2, 5, 6, 16, 17, 33, 64)
SINGLE = (lg.FAMILY_AUTO, lg.FAMILY_ROWS_PER_WAVE, lg.FAMILY_WAVE_PER_ROW,
          lg.FAMILY_GROUP_PER_ROW, lg.FAMILY_BATCHED, lg.FAMILY_BATCHED_MFMA)
BATCHED = (lg.FAMILY_AUTO, lg.FAMILY_BATCHED, lg.FAMILY_BATCHED_MFMA)
GUARD = 16
CANARY = np.float32(-12345.5)
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Packer:
    """Host arrays laid end to end in one buffer of a stored element type;
    each piece starts 16-byte aligned plus `misalign` elements."""

    def __init__(self, dtype):
        self.dtype = dtype
        self.es = gi.ELEMENT_BYTES[dtype] if dtype != "fp32out" else 4
        self.parts, self.size = [], 0

    def add(self, arr, misalign=0):
        per = 16 // self.es
        start = -(-self.size // per) * per + misalign
        self.parts.append((start, np.ascontiguousarray(arr).reshape(-1)))
        self.size = start + arr.size + per
        return start

    def host(self, np_dtype, fill):
        out = np.full(max(self.size, 1), fill, dtype=np_dtype)
        for start, a in self.parts:
            out[start:start + a.size] = a
        return out


def device(dtype, host):
    if dtype == "f32":
        return torch.from_numpy(host.astype(np.float32)).cuda()
    return torch.from_numpy(host.astype(np.uint16).view(np.int16)).view(TORCH[dtype]).cuda()


def run_sweep(dtype, cases, families, nvec_of):
    """cases: list of (M, K, lda, misalign, bias, seed).  Runs every family the
    planner accepts for each case and returns the number of results checked."""
    es = gi.ELEMENT_BYTES[dtype]
    pa, px, pb = Packer(dtype), Packer(dtype), Packer("fp32out")
    specs = []
    for (M, K, lda, mis, bias, seed) in cases:
        nvec = nvec_of(seed)
        c = gi.make_integer(dtype, M, K, seed=seed, nvec=nvec, lda=lda, bias=bias)
        a_off = pa.add(c.A, mis)
        x_off = px.add(c.X, mis)
        b_off = pb.add(c.bias) if bias else None
        specs.append((c, mis, a_off, x_off, b_off))
    # NaN between and around the pieces: a read outside a case's data shows
    nan = gi._padding_value(dtype)
    A = device(dtype, pa.host(gi.storage_dtype(dtype), nan))
    X = device(dtype, px.host(gi.storage_dtype(dtype), nan))
    B = torch.from_numpy(pb.host(np.float32, 0)).cuda()
    a0, x0, b0 = A.data_ptr(), X.data_ptr(), B.data_ptr()

    # plan every (case, family) on the host, lay the outputs out with guards
    runs, out_size = [], GUARD
    for idx, (c, mis, a_off, x_off, b_off) in enumerate(specs):
        A_addr, X_addr = a0 + a_off * es, x0 + x_off * es
        for fam in families:
            try:
                lg.plan(dtype, c.M, c.K, c.lda, c.nvec, A_addr, X_addr, fam)
            except lg.GemvError:
                continue
            runs.append((idx, fam, out_size))
            out_size += c.nvec * c.M + GUARD
    Y = torch.full((out_size,), float(CANARY), dtype=torch.float32, device="cuda")
    y0 = Y.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    for idx, fam, off in runs:
        c, mis, a_off, x_off, b_off = specs[idx]
        bias = b0 + 4 * b_off if b_off is not None else None
        rc = lg.gemv_run_family(lg.DTYPE_CODES[dtype], fam, a0 + a_off * es, c.lda,
                                x0 + x_off * es, bias, y0 + 4 * off, c.M, c.K, c.nvec, stream)
        assert rc == lg.GEMV_SUCCESS, (dtype, c.M, c.K, c.lda, c.nvec, fam, rc)
    torch.cuda.synchronize()
    got = Y.cpu().numpy()

    refs = {}
    mask = np.ones(out_size, dtype=bool)
    for idx, fam, off in runs:
        c, mis = specs[idx][0], specs[idx][1]
        if idx not in refs:
            refs[idx] = oracle.gemv(dtype, c.A, c.X, c.bias, c.M, c.K, lda=c.lda, nvec=c.nvec)[0]
        n = c.nvec * c.M
        y = got[off:off + n].astype(np.float64).reshape(c.nvec, c.M)
        mask[off:off + n] = False
        if not np.array_equal(y, refs[idx]):
            bad = np.argwhere(y != refs[idx])[0]
            raise AssertionError(
                f"{dtype} M={c.M} K={c.K} lda={c.lda} nvec={c.nvec} misalign={mis} "
                f"bias={c.bias is not None} family {lg.FAMILY_NAMES.get(fam, 'auto')}: "
                f"Y[{bad[0]},{bad[1]}] = {y[tuple(bad)]!r}, oracle {refs[idx][tuple(bad)]!r}")
    assert np.all(got[mask] == CANARY), "a write outside an output"
    return len(runs)


@pytest.mark.parametrize("dtype", gi.DTYPES)
def test_tiny_shapes_every_family(dtype):
    cases, seed = [], 0
    for M in M_VALUES:
        for K in K_VALUES:
            for lda, mis in ((K, 0), (K + 1, 0), (K + 8, 0), (K, 1)):
                for bias in (False, True):
                    cases.append((M, K, lda, mis, bias, seed))
                    seed += 1
    n = run_sweep(dtype, cases, SINGLE, lambda s: 1)
    print(f"{dtype}: {len(cases)} shapes, {n} results bit-exact", flush=True)
    assert n >= 3 * len(cases)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiny_shapes_batched(dtype):
    cases, seed = [], 0
    for nvec in NVECS:
        for M in M_VALUES:
            for K in K_BATCHED:
                for lda, mis in ((K, 0), (K + 8, 0), (K + 1, 0)):
                    for bias in (False, True):
                        cases.append((M, K, lda, mis, bias, seed * 100 + nvec))
                        seed += 1
    n = run_sweep(dtype, cases, BATCHED, lambda s: s % 100)
    print(f"{dtype}: {len(cases)} batched shapes, {n} results bit-exact", flush=True)
    assert n >= 2 * len(cases)
