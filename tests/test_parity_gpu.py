"""Parity of libgemv's HIP kernels with the CPU oracle (needs an MI355X).

Every case goes through the C ABI (ctypes), compares element by element with
the fp64 oracle on the same seeded inputs, and checks canary words around
the output.  Integer-valued, identity, one-hot and worked-example inputs
must match bit for bit (every partial sum is exact in fp32, whatever the
order); random inputs must satisfy |y - y_ref| <= 1e-5·Σ|A·x| + 1e-6.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gemv_inputs as gi
import memory_bound_gemv_f32_amd as lg
from gpu_helpers import (assert_bit_exact, assert_within_bound, run_gpu,
                         run_oracle, upload)
from oracle_pins import lib_decode

pytestmark = pytest.mark.gpu

SINGLE_FAMILIES = [lg.FAMILY_AUTO, lg.FAMILY_ROWS_PER_WAVE, lg.FAMILY_WAVE_PER_ROW,
                   lg.FAMILY_GROUP_PER_ROW]


def families_for(case: gi.Case, misalign: int = 0):
    """Every family the planner accepts for this shape and alignment."""
    out = []
    fams = SINGLE_FAMILIES if case.nvec == 1 else [lg.FAMILY_AUTO]
    if case.dtype != "f32":
        fams = fams + [lg.FAMILY_BATCHED, lg.FAMILY_BATCHED_MFMA]
    addr = (1 << 20) + misalign * gi.ELEMENT_BYTES[case.dtype]
    for fam in fams:
        try:
            lg.plan(case.dtype, case.M, case.K, case.lda, case.nvec, addr, addr, fam)
        except lg.GemvError:
            continue
        out.append(fam)
    return out


def pad16(dtype, K):
    per = 16 // gi.ELEMENT_BYTES[dtype]
    return max(per, -(-K // per) * per)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    print(f"device: {torch.cuda.get_device_name(0)} arch {name}", flush=True)


# ---------------------------------------------------------------------------
# bit-exact pins
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", gi.DTYPES)
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("misalign", [0, 1])
def test_worked_example(dtype, bias, misalign):
    """M=3, K=1024 (page "第 3 课：GEMV 与行级并行", section "具体演示与数值推演"):
    y = -512·(m+1) (+ bias), bit-exact on every family that can run it."""
    case = gi.make_worked_example(dtype, bias=bias)
    want = np.array([[-512.0, -1024.0, -1536.0]])
    if bias:
        want = want + np.array([[0.5, -0.25, 1.0]])
    for fam in families_for(case, misalign):
        y = run_gpu(case, fam, misalign=misalign)
        assert_bit_exact(y, want, f"{dtype} family {fam} misalign {misalign}")


@pytest.mark.parametrize("dtype", gi.DTYPES)
@pytest.mark.parametrize("n", [1, 7, 64, 300, 1024, 4096])
def test_identity(dtype, n):
    case = gi.make_identity(dtype, n, seed=n, bias=True)
    ref, _ = run_oracle(case)
    for fam in families_for(case):
        assert_bit_exact(run_gpu(case, fam), ref, f"{dtype} n={n} family {fam}")


@pytest.mark.parametrize("dtype", gi.DTYPES)
@pytest.mark.parametrize("M,K,extra", [(1000, 16, 0), (999, 100, 4), (513, 777, 9),
                                       (300, 4096, 0), (64, 14336, 8)])
def test_one_hot(dtype, M, K, extra):
    case = gi.make_one_hot(dtype, M, K, seed=K, lda=K + extra)
    ref, _ = run_oracle(case)
    for fam in families_for(case):
        assert_bit_exact(run_gpu(case, fam), ref, f"{dtype} {M}x{K} family {fam}")


INT_SHAPES = [(1, 1), (5, 3), (63, 8), (64, 15), (65, 16), (130, 17), (257, 31),
              (33, 32), (17, 33), (9, 127), (300, 128), (31, 129), (7, 255),
              (129, 256), (3, 257), (70, 1000), (40, 1024), (5, 4097), (3, 14337),
              (513, 4200), (515, 8300),  # two rows per workgroup share x
              (300, 1536), (100, 12288), (50, 16384)]  # batches of 3, 6 and 8 loads per lane


@pytest.mark.parametrize("dtype", gi.DTYPES)
@pytest.mark.parametrize("M,K", INT_SHAPES)
def test_integer_every_family(dtype, M, K):
    """Exact-integer regime: every family, with bias, tight and padded row
    pitch, aligned and element-aligned pointers; all bit-exact."""
    for lda, misalign in ((K, 0), (pad16(dtype, K), 0), (K + 3, 0), (pad16(dtype, K), 1)):
        case = gi.make_integer(dtype, M, K, seed=M * 7 + K, lda=lda, bias=True)
        ref, _ = run_oracle(case)
        for fam in families_for(case, misalign):
            y = run_gpu(case, fam, misalign=misalign)
            assert_bit_exact(y, ref, f"{dtype} {M}x{K} lda={lda} misalign={misalign} family {fam}")


# x of 8-24 KiB held in registers while a workgroup walks 2 or 4 rows: 3 to 6
# chunks per lane, the last one whole or partial; the last workgroup short
STREAM_SHAPES = [("bf16", 1025, 8200), ("f16", 513, 12288), ("bf16", 4099, 12288),
                 ("f16", 1030, 10248), ("bf16", 600, 10248), ("f32", 1025, 4100),
                 ("f32", 517, 6144), ("f32", 2051, 6140), ("f32", 1026, 5124),
                 ("bf16", 1025, 4104), ("f16", 600, 6144), ("bf16", 2051, 8192),
                 ("f32", 2050, 2052), ("f32", 777, 3000)]


@pytest.mark.parametrize("dtype,M,K", STREAM_SHAPES)
def test_integer_x_in_registers(dtype, M, K):
    per = 16 // gi.ELEMENT_BYTES[dtype]
    for lda in (K, K + per):
        q = lg.plan(dtype, M, K, lda, 1, 1 << 20, 1 << 20)
        assert q["family"] == lg.FAMILY_GROUP_PER_ROW and q["x_in_registers"] == 1
        case = gi.make_integer(dtype, M, K, seed=M + K, lda=lda, bias=lda == K)
        ref, _ = run_oracle(case)
        print(f"{dtype} {M}x{K} lda={lda}: {q['row_tiles']} rows per workgroup, "
              f"{q['batch']} x chunks per lane", flush=True)
        assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO), ref, f"{dtype} {M}x{K} lda={lda}")


# very many short rows: a wavefront takes 2, 4 or 8 rows; the last
# wavefront's rows run past M
MANY_ROWS_SHAPES = [("bf16", 70001, 264, 2), ("f32", 140001, 132, 4), ("f16", 300003, 264, 8),
                    ("bf16", 140000, 1024, 4)]


@pytest.mark.parametrize("dtype,M,K,tiles", MANY_ROWS_SHAPES)
def test_integer_many_short_rows(dtype, M, K, tiles):
    per = 16 // gi.ELEMENT_BYTES[dtype]
    for lda in (K, K + per):
        q = lg.plan(dtype, M, K, lda, 1, 1 << 20, 1 << 20)
        assert (q["family"], q["row_tiles"]) == (lg.FAMILY_WAVE_PER_ROW, tiles)
        case = gi.make_integer(dtype, M, K, seed=M + K, lda=lda, bias=lda == K)
        ref, _ = run_oracle(case)
        print(f"{dtype} {M}x{K} lda={lda}: {q['row_tiles']} rows per wavefront, "
              f"{q['batch']} loads per lane", flush=True)
        assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO), ref, f"{dtype} {M}x{K} lda={lda}")


# very tall matrices of rows of a load count that is not a power of two: 8
# lanes per row with several loads each (ragged last wavefront, bias on half
# the cases)
SPLIT_LANE_SHAPES = [("f32", 524301, 80, 8), ("bf16", 524301, 160, 8), ("f16", 530001, 176, 8)]


@pytest.mark.parametrize("dtype,M,K,lanes", SPLIT_LANE_SHAPES)
def test_integer_split_lane_rows(dtype, M, K, lanes):
    per = 16 // gi.ELEMENT_BYTES[dtype]
    for lda in (K, K + 1):
        q = lg.plan(dtype, M, K, lda, 1, 1 << 20, 1 << 20)
        assert (q["family"], q["lanes_per_row"]) == (lg.FAMILY_ROWS_PER_WAVE, lanes), q
        assert q["batch"] > 1
        case = gi.make_integer(dtype, M, K, seed=M + 3 * K, lda=lda, bias=lda != K)
        ref, _ = run_oracle(case)
        what = f"{dtype} {M}x{K} lda={lda}: {lanes} lanes x {q['batch']} loads per row"
        print(what, flush=True)
        assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO), ref, what)


# few long rows: workgroups of 16 wavefronts (one row) or 8 (two rows, the
# last pair of an odd M half past the end); rows with and without a ragged
# tail shorter than a 16-byte load
WIDE_SHAPES = [("bf16", 192, 65536, 16), ("f32", 255, 20001, 16), ("f16", 300, 33000, 16),
               ("f16", 511, 24600, 8), ("bf16", 999, 17001, 8), ("f32", 600, 12000, 8)]


@pytest.mark.parametrize("dtype,M,K,waves", WIDE_SHAPES)
def test_integer_wide_workgroups(dtype, M, K, waves):
    per = 16 // gi.ELEMENT_BYTES[dtype]
    for lda, misalign in ((K, 0), (K + per, 0), (K + 1, 1)):
        A_addr = 1 << 20 if misalign == 0 else (1 << 20) + gi.ELEMENT_BYTES[dtype]
        q = lg.plan(dtype, M, K, lda, 1, A_addr, A_addr)
        assert q["family"] == lg.FAMILY_GROUP_PER_ROW and q["waves_per_group"] == waves, q
        case = gi.make_integer(dtype, M, K, seed=M * 7 + K, lda=lda, bias=lda == K)
        ref, _ = run_oracle(case)
        what = (f"{dtype} {M}x{K} lda={lda} misalign={misalign}: {waves} wavefronts, "
                f"{q['row_tiles']} rows, batch {q['batch']}")
        print(what, flush=True)
        assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO, misalign=misalign), ref, what)


# one row per wavefront in workgroups of two wavefronts (a grid that spreads
# more evenly over the compute units than one of four-wavefront workgroups):
# an odd row count leaves the last workgroup one row past the end; rows with
# and without a ragged tail, tight and padded pitches
NARROW_SHAPES = [("bf16", 1535, 4096), ("f16", 2560, 4100), ("f32", 1536, 2050),
                 ("bf16", 1280, 3000)]


@pytest.mark.parametrize("dtype,M,K", NARROW_SHAPES)
def test_integer_two_wavefront_workgroups(dtype, M, K):
    per = 16 // gi.ELEMENT_BYTES[dtype]
    for lda in (K, pad16(dtype, K) + per):
        q = lg.plan(dtype, M, K, lda, 1, 1 << 20, 1 << 20)
        assert (q["family"], q["waves_per_group"], q["grid"]) == \
            (lg.FAMILY_WAVE_PER_ROW, 2, (M + 1) // 2), q
        case = gi.make_integer(dtype, M, K, seed=M * 5 + K, lda=lda, bias=lda == K)
        ref, _ = run_oracle(case)
        for fam in (lg.FAMILY_AUTO, lg.FAMILY_WAVE_PER_ROW):
            what = f"{dtype} {M}x{K} lda={lda} family {fam}: 2 wavefronts, batch {q['batch']}"
            print(what, flush=True)
            assert_bit_exact(run_gpu(case, fam), ref, what)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nvec", list(range(1, 17)))
def test_integer_batched(dtype, nvec):
    for M, K, lda in ((67, 512, 512), (130, 1000, 1000), (9, 4104, 4104), (33, 77, 80)):
        case = gi.make_integer(dtype, M, K, seed=nvec * 100 + K, nvec=nvec, lda=lda,
                               bias=nvec % 2 == 0)
        ref, _ = run_oracle(case)
        y = run_gpu(case, lg.FAMILY_AUTO, batched=True)
        assert_bit_exact(y, ref, f"{dtype} nvec={nvec} {M}x{K}")
        y1 = run_gpu(case, lg.FAMILY_BATCHED, batched=True, misalign=1)
        assert_bit_exact(y1, ref, f"{dtype} nvec={nvec} {M}x{K} element loads")
        y2 = run_gpu(case, lg.FAMILY_BATCHED, batched=True)
        assert_bit_exact(y2, ref, f"{dtype} nvec={nvec} {M}x{K} vector ALU")
        if K % 8 == 0 and lda % 8 == 0:
            y3 = run_gpu(case, lg.FAMILY_BATCHED_MFMA, batched=True)
            assert_bit_exact(y3, ref, f"{dtype} nvec={nvec} {M}x{K} matrix cores")


def test_empty_reduction_gives_bias():
    for dtype in gi.DTYPES:
        for bias in (False, True):
            case = gi.make_integer(dtype, 100, 0, seed=1, bias=bias)
            want = case.bias.astype(np.float64)[None, :] if bias else np.zeros((1, 100))
            for fam in families_for(case):
                assert_bit_exact(run_gpu(case, fam), want, f"K=0 {dtype} family {fam}")


def test_nan_stays_in_its_row():
    for dtype in gi.DTYPES:
        case = gi.make_random(dtype, 300, 1000, seed=3, lda=1000)
        nan = gi.quantise(dtype, np.array([np.nan]))[0]
        case.A = case.A.copy()
        case.A[123, 456] = nan
        for fam in families_for(case):
            y = run_gpu(case, fam)[0]
            assert np.isnan(y[123]), (dtype, fam)
            assert np.all(np.isfinite(np.delete(y, 123))), (dtype, fam)


def test_f16_subnormals_are_kept():
    """fp16 subnormal A (2^-20 · small integers) times integer x: exact sums."""
    rng = np.random.default_rng(5)
    M, K = 256, 4096
    a = rng.integers(-7, 8, size=(M, K)) * 2.0 ** -20
    x = rng.integers(-7, 8, size=(1, K)).astype(np.float64)
    case = gi.Case("sub_f16", "f16", M, K, gi.quantise("f16", a), gi.quantise("f16", x), None, K)
    ref, _ = run_oracle(case)
    for fam in families_for(case):
        assert_bit_exact(run_gpu(case, fam), ref, f"subnormal family {fam}")
    case.nvec = 4
    case.X = gi.quantise("f16", np.repeat(x, 4, axis=0))
    ref, _ = run_oracle(case)
    assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO, batched=True), ref, "subnormal batched")


# ---------------------------------------------------------------------------
# random data within the bound
# ---------------------------------------------------------------------------

RANDOM_SHAPES = [(1, 5), (777, 16), (1000, 37), (513, 128), (100, 255), (257, 1000),
                 (2048, 4096), (1024, 4096), (31, 14336), (4097, 300)]


@pytest.mark.parametrize("dtype", gi.DTYPES)
@pytest.mark.parametrize("M,K", RANDOM_SHAPES)
def test_random_every_family(dtype, M, K):
    for lda in (K, pad16(dtype, K) + 8):
        case = gi.make_random(dtype, M, K, seed=M + K, lda=lda, bias=True, dist="normal")
        ref, absdot = run_oracle(case)
        for fam in families_for(case):
            y = run_gpu(case, fam)
            assert_within_bound(y, ref, absdot, f"{dtype} {M}x{K} lda={lda} family {fam}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nvec", [17, 24, 31, 32, 33, 47, 64])
def test_integer_wide_batched(dtype, nvec):
    """17-64 vectors: one pass over A on the matrix cores (2 or 4 vector
    tiles), or blocks of 16 vectors on the vector ALUs; all bit-exact."""
    for M, K, lda in ((67, 512, 512), (130, 1000, 1000), (9, 4104, 4104), (33, 77, 80),
                      (300, 2048, 2056)):
        case = gi.make_integer(dtype, M, K, seed=nvec * 100 + K, nvec=nvec, lda=lda,
                               bias=nvec % 2 == 1)
        ref, _ = run_oracle(case)
        assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO, batched=True), ref,
                         f"{dtype} nvec={nvec} {M}x{K}")
        assert_bit_exact(run_gpu(case, lg.FAMILY_BATCHED, batched=True, misalign=1), ref,
                         f"{dtype} nvec={nvec} {M}x{K} element loads")
        assert_bit_exact(run_gpu(case, lg.FAMILY_BATCHED, batched=True), ref,
                         f"{dtype} nvec={nvec} {M}x{K} vector ALU blocks")
        if K % 8 == 0 and lda % 8 == 0:
            assert_bit_exact(run_gpu(case, lg.FAMILY_BATCHED_MFMA, batched=True), ref,
                             f"{dtype} nvec={nvec} {M}x{K} matrix cores")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,nvec", [(2049, 3), (2049, 4), (3001, 2), (3001, 17), (4089, 2),
                                    (4087, 5), (5003, 16), (1025, 33)])
def test_integer_batched_row_counts(dtype, M, nvec):
    """The vector-ALU batched kernels with one and with two rows per
    wavefront, on row counts either side of the switch between them and not
    a multiple of a workgroup's rows (17 and 33 vectors: blocks of 16 and a
    remainder, each planned on its own); aligned and unaligned rows."""
    for K, lda in ((4100, 4100), (4100, 4104), (1000, 1000)):
        case = gi.make_integer(dtype, M, K, seed=M + nvec + K, nvec=nvec, lda=lda, bias=True)
        ref, _ = run_oracle(case)
        q = lg.plan(dtype, M, K, lda, nvec, 1 << 20, 1 << 20, family=lg.FAMILY_BATCHED)
        what = f"{dtype} {M}x{K} lda={lda} nvec={nvec}, {q['rows_per_wave']} rows per wavefront"
        print(what, flush=True)
        assert_bit_exact(run_gpu(case, lg.FAMILY_BATCHED, batched=True), ref, what)
        assert_bit_exact(run_gpu(case, lg.FAMILY_BATCHED, batched=True, misalign=1), ref,
                         what + ", element loads")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nvec", [2, 9, 16, 17])
def test_integer_batched_k_split(dtype, nvec):
    """Up to 512 rows the vector-ALU batched kernel splits each row's K over
    the workgroup's 4 wavefronts, up to 1536 rows (4 or more vectors) over
    pairs of wavefronts: row lengths that give some wavefronts no batch, a
    partial last batch, an element-wise tail, a last workgroup with one row
    group; 16-byte and element loads; bias or none; bit-exact.  Then long
    random rows within the bound."""
    for M, K in ((1, 7), (5, 1000), (64, 4100), (511, 2056), (512, 14337), (3, 16392),
                 (513, 4100), (1023, 2050), (1536, 1000)):
        case = gi.make_integer(dtype, M, K, seed=M * 7 + K + nvec, nvec=nvec, bias=(M + nvec) % 2 == 1)
        ref, _ = run_oracle(case)
        q = lg.plan(dtype, M, K, K, nvec, 1 << 20, 1 << 20, family=lg.FAMILY_BATCHED)
        ks = 4 if M <= 512 else (2 if nvec >= 4 else 1)  # wavefronts per row
        assert q["lanes_per_row"] == 64 * ks, q
        what = f"{dtype} {M}x{K} nvec={nvec}: K split over {ks} wavefronts"
        print(what, flush=True)
        assert_bit_exact(run_gpu(case, lg.FAMILY_BATCHED, batched=True), ref, what)
        assert_bit_exact(run_gpu(case, lg.FAMILY_BATCHED, batched=True, misalign=1), ref,
                         what + ", element loads")
    case = gi.make_random(dtype, 64, 100003, seed=nvec, nvec=nvec, bias=True, dist="normal",
                          scale=1 / 256)
    ref, absdot = run_oracle(case)
    assert_within_bound(run_gpu(case, lg.FAMILY_AUTO, batched=True), ref, absdot,
                        f"{dtype} 64x100003 nvec={nvec} random, K split")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nvec", [2, 3, 8, 13, 16, 20, 32, 64])
def test_random_batched(dtype, nvec):
    for M, K in ((4096, 4096), (1000, 1000), (64, 14336)):
        case = gi.make_random(dtype, M, K, seed=nvec + K, nvec=nvec, bias=True,
                              dist="normal", scale=1 / np.sqrt(K))
        ref, absdot = run_oracle(case)
        for fam in (lg.FAMILY_AUTO, lg.FAMILY_BATCHED, lg.FAMILY_BATCHED_MFMA):
            y = run_gpu(case, fam, batched=True)
            assert_within_bound(y, ref, absdot, f"{dtype} nvec={nvec} {M}x{K} family {fam}")


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_scaling_negation_permutation_determinism():
    for dtype in gi.DTYPES:
        case = gi.make_random(dtype, 1111, 3000, seed=9, dist="normal")
        y = run_gpu(case, lg.FAMILY_AUTO)
        assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO), y, "repeat")
        # doubling and negating are exact in every encoding at these magnitudes
        X2 = gi.quantise(dtype, 2.0 * lib_decode(dtype, case.X))
        Xn = gi.quantise(dtype, -1.0 * lib_decode(dtype, case.X))
        for X, factor in ((X2, 2.0), (Xn, -1.0)):
            c2 = gi.Case(case.name, dtype, case.M, case.K, case.A, X.astype(case.X.dtype),
                         None, case.lda)
            assert_bit_exact(run_gpu(c2, lg.FAMILY_AUTO), factor * y, f"{dtype} x*{factor}")
        perm = np.random.default_rng(1).permutation(case.M)
        cp = gi.Case(case.name, dtype, case.M, case.K, case.A[perm], case.X, None, case.lda)
        assert_bit_exact(run_gpu(cp, lg.FAMILY_AUTO), y[:, perm], f"{dtype} row permutation")


def test_batched_columns_and_single_vector_agree():
    for dtype in ("f16", "bf16"):
        case = gi.make_random(dtype, 2000, 2048, seed=4, nvec=11, bias=True, dist="normal")
        Y = run_gpu(case, lg.FAMILY_AUTO, batched=True)
        ref, absdot = run_oracle(case)
        assert_within_bound(Y, ref, absdot, "batched")
        perm = np.random.default_rng(2).permutation(case.nvec)
        cp = gi.Case(case.name, dtype, case.M, case.K, case.A, case.X[perm], case.bias,
                     case.lda, case.nvec)
        assert_bit_exact(run_gpu(cp, lg.FAMILY_AUTO, batched=True), Y[perm], "column permutation")
        # 40 vectors span three matrix-core tiles: columns moved between tiles
        # (and into the zero-padded last tile) give the same bits
        wide = gi.make_random(dtype, 500, 1024, seed=5, nvec=40, bias=True, dist="normal")
        W = run_gpu(wide, lg.FAMILY_AUTO, batched=True)
        perm = np.random.default_rng(3).permutation(wide.nvec)
        cw = gi.Case(wide.name, dtype, wide.M, wide.K, wide.A, wide.X[perm], wide.bias,
                     wide.lda, wide.nvec)
        assert_bit_exact(run_gpu(cw, lg.FAMILY_AUTO, batched=True), W[perm],
                         "column permutation across tiles")
        for j in (0, 5, 10):
            c1 = gi.Case(case.name, dtype, case.M, case.K, case.A, case.X[j:j + 1], case.bias,
                         case.lda)
            assert_within_bound(run_gpu(c1, lg.FAMILY_AUTO), ref[j:j + 1], absdot[j:j + 1],
                                f"single vector {j}")


# ---------------------------------------------------------------------------
# the full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(gi.WORKLOADS))
def test_full_size_workload(name):
    case = gi.make_workload(name)
    print(f"workload {name}: {case.dtype} M={case.M} K={case.K} nvec={case.nvec}", flush=True)
    ref, absdot = run_oracle(case)
    y = run_gpu(case, lg.FAMILY_AUTO, batched=case.nvec > 1)
    assert_within_bound(y, ref, absdot, name)


def test_read_probe_reads_and_writes_nothing():
    """The measurement probe streams a buffer (whole and ragged sizes) and
    leaves the sink word alone."""
    buf = torch.full(((3 << 20) // 4 + 64,), 0x01010101, dtype=torch.int32, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    for nbytes in (16, 1040, 1 << 20, (3 << 20) + 16):
        rc = lg.gemv_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
        assert rc == lg.GEMV_SUCCESS
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [7, 7, 7, 7]


def test_read_probe_variants_write_only_timestamps():
    """Every read-pattern variant streams the buffer and writes nothing but
    its per-wavefront timestamps (start <= end, every wavefront's pair
    written, entries past them untouched)."""
    buf = torch.full(((2 << 20) // 4,), 0x01010101, dtype=torch.int32, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for loads, waves, blocks, flags in ((8, 4, 1, 0), (2, 16, 1, 1), (16, 1, 3, 4), (4, 8, 2, 6),
                                        (8, 2, 1, 3)):
        per_wave = loads * 1024 * blocks
        n_waves = -(-buf.numel() * 4 // per_wave)
        n_waves = -(-n_waves // waves) * waves
        times = torch.full((2 * n_waves + 8,), -1, dtype=torch.int64, device="cuda")
        rc = lg.gemv_read_probe_variant(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), loads,
                                        waves, blocks, flags, times.data_ptr(), times.numel(),
                                        stream)
        assert rc == lg.GEMV_SUCCESS
        torch.cuda.synchronize()
        t = times.cpu().numpy()
        pairs = t[:2 * n_waves].reshape(n_waves, 2)
        assert np.all(pairs >= 0) and np.all(pairs[:, 1] >= pairs[:, 0]), (loads, waves, blocks)
        assert np.all(t[2 * n_waves:] == -1)
    assert sink.cpu().tolist() == [7, 7, 7, 7]


def test_seeded_random_shapes_integer():
    """Sixty shapes drawn from a fixed seed (M, K, row pitch, pointer
    offset, bias, dtype, family, batch size), all in the exact-integer
    regime: every result bit-exact."""
    rng = np.random.default_rng(2024)
    for trial in range(60):
        dtype = str(rng.choice(gi.DTYPES))
        M = int(rng.choice([1, 2, 3, 7, 63, 64, 65, 255, 256, 257, 1000, 3000, 9000]))
        K = int(rng.choice([1, 5, 8, 16, 31, 64, 100, 129, 512, 1000, 2049, 4096, 7000, 16384]))
        per = 16 // gi.ELEMENT_BYTES[dtype]
        lda = K + int(rng.choice([0, 0, 1, per, 3 * per + 1]))
        misalign = int(rng.choice([0, 0, 1]))
        nvec = 1 if dtype == "f32" else int(rng.choice([1, 1, 2, 5, 16, 24]))
        case = gi.make_integer(dtype, M, K, seed=trial, nvec=nvec, lda=lda,
                               bias=bool(rng.integers(2)))
        ref, _ = run_oracle(case)
        fams = families_for(case, misalign)
        fam = fams[int(rng.integers(len(fams)))]
        y = run_gpu(case, fam, misalign=misalign, batched=nvec > 1)
        assert_bit_exact(y, ref, f"trial {trial}: {dtype} {M}x{K} lda={lda} nvec={nvec} "
                                 f"misalign={misalign} family {fam}")


def test_seeded_random_shapes_automatic_plan():
    """A hundred shapes drawn from a fixed seed around the automatic planner's
    boundaries (row counts near 256, 512, 6144 and the row-tile thresholds;
    rows of 16 bytes to 32 KiB, x just below and above 8, 16 and 24 KiB; odd
    row pitches and offsets), each run through the planner's own choice of
    kernel: every result bit-exact."""
    import memory_bound_gemv_f32_amd as lg
    rng = np.random.default_rng(4242)
    row_counts = [1, 3, 255, 256, 257, 510, 511, 512, 1023, 6143, 6144, 6145, 16383,
                  65537, 131071, 262147]
    row_bytes = [16, 48, 256, 512, 520, 1024, 2048, 4096, 8192, 8208, 12288, 16384, 16400,
                 24576, 24592, 28672, 32768]
    done = 0
    while done < 100:
        dtype = str(rng.choice(gi.DTYPES))
        es = gi.ELEMENT_BYTES[dtype]
        M = int(rng.choice(row_counts))
        K = int(rng.choice(row_bytes)) // es + int(rng.choice([0, 0, 0, 0, 0, 1, -1]))
        if K < 1 or M * K > 36_000_000:
            continue
        per = 16 // es
        lda = K + int(rng.choice([0, 0, 0, 1, per]))
        misalign = int(rng.choice([0, 0, 0, 0, 1]))
        case = gi.make_integer(dtype, M, K, seed=1000 + done, lda=lda, bias=bool(rng.integers(2)))
        A_addr = 1 << 20 if misalign == 0 else (1 << 20) + es
        q = lg.plan(dtype, M, K, lda, 1, A_addr, A_addr)
        what = (f"trial {done}: {dtype} {M}x{K} lda={lda} misalign={misalign}: family "
                f"{lg.FAMILY_NAMES[q['family']]}, batch {q['batch']}, tiles {q['row_tiles']}")
        print(what, flush=True)
        ref, _ = run_oracle(case)
        assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO, misalign=misalign), ref, what)
        done += 1


# the lengths whose last, partial 64-element step the matrix-core kernel
# once dropped (K % 8 == 0, K % 64 != 0, 7·ceil(steps/8) > steps), and
# neighbours; every vector-tile count
MFMA_TAIL_K = [8, 72, 120, 136, 200, 392, 600, 840, 1096, 1608, 2120, 2632, 2680]
MFMA_TAIL_NVEC = [2, 5, 6, 16, 17, 32, 33, 64]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nvec", MFMA_TAIL_NVEC)
def test_integer_batched_partial_last_step(dtype, nvec):
    for K in MFMA_TAIL_K:
        case = gi.make_integer(dtype, 33, K, seed=K + nvec, nvec=nvec, bias=K % 16 == 8)
        ref, _ = run_oracle(case)
        q = lg.plan(dtype, case.M, K, K, nvec, 1 << 20, 1 << 20)
        assert q["family"] == lg.FAMILY_BATCHED_MFMA, q
        for fam in (lg.FAMILY_AUTO, lg.FAMILY_BATCHED_MFMA):
            assert_bit_exact(run_gpu(case, fam, batched=True), ref,
                             f"{dtype} 33x{K} nvec={nvec} family {fam}")


# matrix-core workgroup shapes: (rows, wavefronts, row groups, rows per
# workgroup).  Up to 1024 rows one group of 4, up to 2048 one group of 8;
# more 16-row tiles than compute units: 4 wavefronts, each walking two chunks
# and the leftover steps of its longer K run.  Every row count leaves the
# last workgroup partly past the end.
MFMA_GEOMETRIES = [(1021, 8, 1, 4), (1031, 8, 1, 8), (2057, 8, 2, 16), (4113, 4, 2, 16)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,waves,groups,rows", MFMA_GEOMETRIES)
def test_integer_batched_workgroup_shapes(dtype, M, waves, groups, rows):
    for K, nvec in ((4096, 3), (4096, 16), (1000, 33), (2680, 17)):
        q = lg.plan(dtype, M, K, K, nvec, 1 << 20, 1 << 20)
        assert q["family"] == lg.FAMILY_BATCHED_MFMA, q
        want = 8 if rows == 4 and nvec <= 5 else rows  # 4-row groups: X staged in LDS only
        assert (q["waves_per_group"], q["row_tiles"], q["rows_per_group"]) == (waves, groups, want), q
        case = gi.make_integer(dtype, M, K, seed=K + nvec, nvec=nvec, bias=nvec % 2 == 1)
        ref, _ = run_oracle(case)
        what = f"{dtype} {M}x{K} nvec={nvec}: {waves} wavefronts, {groups} row groups, chunk {q['batch']}"
        print(what, flush=True)
        assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO, batched=True), ref, what)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_integer_batched_four_row_groups(dtype):
    """6-16 vectors on tall matrices: workgroups of four 8-row groups (32
    rows, 4 wavefronts, chunks of 4 steps), on row counts that leave a
    partial last workgroup, K that leave a partial last 64-wide step or
    steps outside whole chunks, bias or none, odd M (unaligned Y columns);
    bit-exact.  Then random data within the bound."""
    for M, K, nvec in ((13313, 4096, 9), (13313, 4096, 16), (14337, 1000, 12), (16384, 2680, 16),
                       (13320, 4104, 13), (14336, 4096, 6), (13313, 1000, 8)):
        q = lg.plan(dtype, M, K, K, nvec, 1 << 20, 1 << 20)
        assert (q["family"], q["row_tiles"], q["rows_per_group"], q["waves_per_group"]) == \
            (lg.FAMILY_BATCHED_MFMA, 4, 32, 4), q
        case = gi.make_integer(dtype, M, K, seed=M + K + nvec, nvec=nvec, bias=nvec % 2 == 1)
        ref, _ = run_oracle(case)
        what = f"{dtype} {M}x{K} nvec={nvec}: four row groups, chunk {q['batch']}"
        print(what, flush=True)
        assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO, batched=True), ref, what)
    case = gi.make_random(dtype, 14336, 4096, seed=7, nvec=16, bias=True, dist="normal",
                          scale=1 / 64)
    ref, absdot = run_oracle(case)
    assert_within_bound(run_gpu(case, lg.FAMILY_AUTO, batched=True), ref, absdot,
                        f"{dtype} 14336x4096 nvec=16 random, four row groups")


def test_refused_launch_reports_launch_failure():
    """A launch the runtime refuses comes back as GEMV_ERROR_LAUNCH_FAILURE
    with the runtime's error code, and leaves nothing behind: the runtime's
    last error is cleared, so torch and later calls work as before."""
    stream = torch.cuda.current_stream().cuda_stream
    assert lg.gemv_test_refused_launch(stream) == lg.GEMV_ERROR_LAUNCH_FAILURE
    code = lg.gemv_last_hip_error()
    name = lg.gemv_last_hip_error_string().decode()
    print(f"refused launch: hipError {code} ({name})", flush=True)
    assert code != 0 and name.startswith("hip")
    err = lg.GemvError(lg.GEMV_ERROR_LAUNCH_FAILURE, "gemv_test_refused_launch")
    assert name in str(err)
    t = torch.arange(1000, dtype=torch.float32, device="cuda") * 2
    torch.cuda.synchronize()
    assert float(t.sum()) == 999000.0
    case = gi.make_integer("bf16", 100, 300, seed=3, bias=True)
    ref, _ = run_oracle(case)
    assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO), ref, "after a refused launch")


@pytest.mark.parametrize("dtype", gi.DTYPES)
def test_long_rows_of_positive_terms_within_bound(dtype):
    """All-positive A and x (no cancellation: rounding errors all push the
    same way) on rows of 2^20 elements, every family that takes them and
    split-K: every output within 1e-5·Σ|A·x| + 1e-6, as the plans'
    rounding-chain bound promises."""
    M, K = 24, 1 << 20
    rng = np.random.default_rng(77)
    a = rng.uniform(0.0, 1.0, size=(M, K))
    x = rng.uniform(0.0, 1.0, size=(1, K))
    case = gi.Case("pos", dtype, M, K, gi.quantise(dtype, a), gi.quantise(dtype, x), None, K)
    ref, absdot = run_oracle(case)
    for fam in families_for(case):
        q = lg.plan(dtype, M, K, K, 1, 1 << 20, 1 << 20, fam)
        y = run_gpu(case, fam)
        err = np.abs(y - ref) / (1e-5 * absdot + 1e-6)
        print(f"{dtype} {M}x{K} family {fam}: chain {q['rounding_chain']}, "
              f"worst error / bound {err.max():.3g}", flush=True)
        assert_within_bound(y, ref, absdot, f"{dtype} positive {M}x{K} family {fam}")
    A, X, _ = upload(case)
    y = lg.gemv_splitk(A, X[0]).cpu().numpy().astype(np.float64)[None, :]
    assert_within_bound(y, ref, absdot, f"{dtype} positive {M}x{K} split-K")
    if dtype != "f32":
        Kb = 1 << 17
        bc = gi.Case("posb", dtype, 64, Kb, gi.quantise(dtype, rng.uniform(0, 1, (64, Kb))),
                     gi.quantise(dtype, rng.uniform(0, 1, (40, Kb))), None, Kb, 40)
        refb, absb = run_oracle(bc)
        for fam in (lg.FAMILY_AUTO, lg.FAMILY_BATCHED):
            assert_within_bound(run_gpu(bc, fam, batched=True), refb, absb,
                                f"{dtype} positive 64x{Kb} nvec=40 family {fam}")

