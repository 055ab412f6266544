"""Parity of weight-only int8 GEMV (gemv_q8_*) with the CPU oracle (needs a
GPU): y = scale ⊙ (Q·x) (+ bias) with int8 Q, fp32 per-row scales and x in
fp32, fp16 or bf16.  Integer inputs with power-of-two scales are bit-exact on
every family, row pitch and alignment; random inputs satisfy
|y - y_ref| <= 1e-5·|scale|·Σ|Q·x| + 1e-6; canary words around y are never
written."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gemv_inputs as gi
import memory_bound_gemv_f32_amd as lg
import oracle
from gpu_helpers import (assert_bit_exact, assert_within_bound, check_guards, guarded_out,
                         to_device)

pytestmark = pytest.mark.gpu

FAMILIES = [lg.FAMILY_AUTO, lg.FAMILY_ROWS_PER_WAVE, lg.FAMILY_WAVE_PER_ROW,
            lg.FAMILY_GROUP_PER_ROW]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def families_for(case: gi.Q8Case, misalign: int = 0):
    """Every family the planner accepts for this shape and alignment."""
    q_addr = (1 << 20) + misalign
    x_addr = (1 << 20) + misalign * gi.ELEMENT_BYTES[case.xdtype]
    out = []
    for fam in FAMILIES:
        try:
            lg.plan_q8(case.xdtype, case.M, case.K, case.ldq, q_addr, x_addr, fam)
        except lg.GemvError:
            continue
        out.append(fam)
    return out


def upload_q8(case: gi.Q8Case, misalign: int = 0):
    """Device Q (an (M, K) view with row stride ldq, starting ``misalign``
    bytes into its allocation), scale, x (``misalign`` elements in) and bias."""
    flat = torch.from_numpy(np.ascontiguousarray(case.Q).reshape(-1))
    buf = torch.empty(flat.numel() + misalign + 16, dtype=torch.int8, device="cuda")
    Qd = buf[misalign:misalign + flat.numel()]
    Qd.copy_(flat)
    Q = Qd.view(case.M, case.ldq)[:, :case.K]
    x = to_device(case.xdtype, case.X.reshape(case.nvec, case.K), misalign)[0]
    scale = torch.from_numpy(case.scale.astype(np.float32)).cuda()
    bias = None if case.bias is None else torch.from_numpy(case.bias.astype(np.float32)).cuda()
    return Q, scale, x, bias


def run_q8(case: gi.Q8Case, family: int = lg.FAMILY_AUTO, misalign: int = 0):
    """y as float64 (1, M); checks the canaries around y."""
    Q, scale, x, bias = upload_q8(case, misalign)
    buf, out = guarded_out((case.M,))
    lg.gemv_q8(Q, scale, x, bias, out=out, family=family)
    torch.cuda.synchronize()
    check_guards(buf, case.M)
    return out.cpu().numpy().astype(np.float64)[None, :]


def run_oracle_q8(case: gi.Q8Case):
    return oracle.gemv_q8(case.xdtype, case.Q, case.scale, case.X, case.bias, case.M, case.K,
                          ldq=case.ldq, nvec=case.nvec)


@pytest.mark.parametrize("xdtype", gi.DTYPES)
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("misalign", [0, 1])
def test_worked_example(xdtype, bias, misalign):
    """M=3, K=1024 walk-through with int8 weights (m+1)(-1)^k and scales
    2^-(m+1): y = [-256, -256, -192] (+ bias) on every family."""
    case = gi.make_q8_worked_example(xdtype, bias=bias)
    want = np.array([[-256.0, -256.0, -192.0]])
    if bias:
        want = want + np.array([[0.5, -0.25, 1.0]])
    for fam in families_for(case, misalign):
        assert_bit_exact(run_q8(case, fam, misalign), want,
                         f"{xdtype} family {fam} misalign {misalign}")


INT_SHAPES = [(1, 1), (5, 3), (63, 15), (64, 16), (65, 17), (130, 31), (257, 32), (33, 33),
              (9, 127), (300, 128), (31, 129), (7, 255), (129, 256), (3, 257), (70, 1000),
              (40, 1024), (1000, 64), (5, 4097), (3, 14337), (2100, 512)]


@pytest.mark.parametrize("xdtype", gi.DTYPES)
@pytest.mark.parametrize("M,K", INT_SHAPES)
def test_integer_every_family(xdtype, M, K):
    """Exact-integer regime (every int8 value, integer x in [-8, 8],
    power-of-two scales, integer bias): bit-exact for every family, tight
    and padded row pitch, aligned and byte-aligned Q."""
    for ldq, misalign in ((K, 0), (-(-K // 16) * 16, 0), (K + 3, 0), (-(-K // 16) * 16, 1)):
        case = gi.make_q8_integer(xdtype, M, K, seed=M * 7 + K, ldq=ldq, bias=True)
        ref, _ = run_oracle_q8(case)
        for fam in families_for(case, misalign):
            assert_bit_exact(run_q8(case, fam, misalign), ref,
                             f"{xdtype} {M}x{K} ldq={ldq} misalign={misalign} family {fam}")


@pytest.mark.parametrize("xdtype", gi.DTYPES)
def test_integer_two_rows_per_workgroup(xdtype):
    """Workgroups of two int8 rows sharing each x chunk (more than 4096
    rows, or an x row of 16 KiB or more): an odd row count leaves the last
    workgroup one row, and a row length that is not a whole number of
    16-byte loads leaves a tail; bit-exact with padded and tight pitches."""
    shapes = [(4099, 4100, 4112), (4099, 4096, 4096), (16383, 4096, 4096)]
    if xdtype == "f32":
        shapes.append((2049, 4096, 4096))  # two rows for the 16 KiB x row alone
    for M, K, ldq in shapes:
        q = lg.plan_q8(xdtype, M, K, ldq, 1 << 20, 1 << 20)
        # (a 16 KiB fp32 x row of whole loads is kept in registers over 4 rows)
        rows = 4 if q["x_in_registers"] else 2
        assert q["x_in_registers"] == (xdtype == "f32" and K % 16 == 0), (M, K, q)
        assert q["family"] == lg.FAMILY_GROUP_PER_ROW and q["row_tiles"] == rows, (M, K, q)
        case = gi.make_q8_integer(xdtype, M, K, seed=M + K + ldq, ldq=ldq, bias=True)
        ref, _ = run_oracle_q8(case)
        assert_bit_exact(run_q8(case), ref, f"{xdtype} {M}x{K} ldq={ldq}")


@pytest.mark.parametrize("xdtype", gi.DTYPES)
def test_integer_x_in_registers(xdtype):
    """int8 rows with x kept in registers while a workgroup walks 2 or 4 of
    them: 1 to 4 x chunks per lane (3 with fp32 x), the last partly past the
    row, a last workgroup with fewer rows, padded pitches, bias or none;
    bit-exact.  Then random data within the bound."""
    shapes = [(4097, 11008, 11008), (1027, 16384, 16400), (4095, 4096 if xdtype == "f32" else 8320, 8336),
              (702, 11008, 11008)]
    if xdtype == "f32":
        shapes = [(4097, 11008, 11008), (1027, 8192, 8208), (4095, 4096, 4112), (702, 12288, 12288)]
    for i, (M, K, ldq) in enumerate(shapes):
        q = lg.plan_q8(xdtype, M, K, ldq, 1 << 20, 1 << 20)
        assert q["family"] == lg.FAMILY_GROUP_PER_ROW and q["x_in_registers"] == 1, (M, K, q)
        case = gi.make_q8_integer(xdtype, M, K, seed=M + K + ldq, ldq=ldq, bias=i % 2 == 0)
        ref, _ = run_oracle_q8(case)
        what = f"{xdtype} {M}x{K} ldq={ldq}: x in registers, {q['batch']} chunks, {q['row_tiles']} rows"
        print(what, flush=True)
        assert_bit_exact(run_q8(case), ref, what)
    case = gi.make_q8_random(xdtype, 2048, 11008, seed=11, bias=True)
    ref, absdot = run_oracle_q8(case)
    assert_within_bound(run_q8(case), ref, absdot, f"{xdtype} 2048x11008 random, x in registers")


RANDOM_SHAPES = [(1000, 16), (4096, 100), (2000, 1000), (513, 4096), (64, 14336),
                 (4096, 4096), (300, 50000)]


@pytest.mark.parametrize("xdtype", gi.DTYPES)
@pytest.mark.parametrize("M,K", RANDOM_SHAPES)
def test_random_every_family(xdtype, M, K):
    case = gi.make_q8_random(xdtype, M, K, seed=M + K, bias=True)
    ref, absdot = run_oracle_q8(case)
    for fam in families_for(case):
        assert_within_bound(run_q8(case, fam), ref, absdot, f"{xdtype} {M}x{K} family {fam}")


def test_edge_cases():
    for xdtype in gi.DTYPES:
        # K = 0: the empty sum, y = bias
        case = gi.make_q8_integer(xdtype, 7, 0, seed=1, bias=True)
        assert_bit_exact(run_q8(case), case.bias[None, :].astype(np.float64), "K=0")
        # a NaN scale reaches its own row only
        case = gi.make_q8_integer(xdtype, 300, 700, seed=2)
        case.scale = case.scale.copy()
        case.scale[123] = np.float32(np.nan)
        y = run_q8(case)[0]
        assert np.isnan(y[123]) and not np.isnan(np.delete(y, 123)).any()
        # scaling x by 2 scales y by 2 exactly; negating x negates y exactly
        case = gi.make_q8_random(xdtype, 1000, 3000, seed=3)
        y = run_q8(case)
        x2 = gi.quantise(xdtype, 2.0 * decode_x(xdtype, case.X))
        xn = gi.quantise(xdtype, -decode_x(xdtype, case.X))
        for X, factor in ((x2, 2.0), (xn, -1.0)):
            other = gi.Q8Case(case.name, xdtype, case.M, case.K, case.Q, case.scale, X, None,
                              case.ldq)
            assert_bit_exact(run_q8(other), factor * y, f"{xdtype} x·{factor}")
    # M = 0 is a no-op
    Q = torch.empty((0, 64), dtype=torch.int8, device="cuda")
    s = torch.empty((0,), dtype=torch.float32, device="cuda")
    x = torch.ones(64, dtype=torch.float16, device="cuda")
    assert lg.gemv_q8(Q, s, x).shape == (0,)


def decode_x(xdtype: str, X: np.ndarray) -> np.ndarray:
    """Stored x back to float64 (fp32 as is, fp16 by numpy, bf16 as the top
    half of an fp32)."""
    if xdtype == "f32":
        return X.astype(np.float64)
    if xdtype == "f16":
        return X.view(np.float16).astype(np.float64)
    return (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_two_calls_bit_identical():
    case = gi.make_q8_random("bf16", 4096, 4096, seed=9)
    assert_bit_exact(run_q8(case), run_q8(case), "two calls")


@pytest.mark.parametrize("name", list(gi.Q8_WORKLOADS))
def test_full_size_q8_workload(name):
    case = gi.make_q8_workload(name)
    print(f"workload {name}: {case.xdtype} M={case.M} K={case.K}", flush=True)
    ref, absdot = run_oracle_q8(case)
    assert_within_bound(run_q8(case), ref, absdot, name)


@pytest.mark.parametrize("xdtype", gi.DTYPES)
def test_integer_tall_rows_of_17_to_24_loads(xdtype):
    """A very tall int8 matrix of 320-byte rows (20 loads): rows of a load
    count that is not a power of two keep one load per lane for int8 weights
    (their rows kernels exist for one load per lane only), bit-exact."""
    M, K = 524301, 320
    q = lg.plan_q8(xdtype, M, K, K, 1 << 20, 1 << 20)
    assert q["family"] == lg.FAMILY_ROWS_PER_WAVE and q["batch"] == 1, q
    case = gi.make_q8_integer(xdtype, M, K, seed=17, bias=True)
    ref, _ = run_oracle_q8(case)
    assert_bit_exact(run_q8(case), ref, f"int8 x {xdtype} {M}x{K}")
