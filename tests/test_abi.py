"""libgemv's C ABI on the host: the library loads, exports what the header
declares, validates arguments before touching the GPU, and maps shapes onto
kernel families as designed.  No GPU and no compute call is needed."""

import ctypes
import json
import re
from pathlib import Path

import pytest

import memory_bound_gemv_f32_amd as lg

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "gemv.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemv_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("gemv_f32", "gemv_f16", "gemv_bf16", "gemv_batched_f16",
                 "gemv_batched_bf16", "gemv_status_string", "gemv_plan",
                 "gemv_run_family"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(lg.LIBRARY))
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) <= set(lg.EXPORTED)


def test_status_strings():
    for code in (lg.GEMV_SUCCESS, lg.GEMV_ERROR_INVALID_VALUE, lg.GEMV_ERROR_LAUNCH_FAILURE):
        assert lg.gemv_status_string(code).startswith(b"GEMV_")
    assert b"unknown" in lg.gemv_status_string(99)


# Invalid arguments are rejected before any HIP call, so these run without a
# GPU.  Pointers here are dummies that must never be dereferenced.
GOOD = 0x10000


@pytest.mark.parametrize("args", [
    dict(M=-1), dict(K=-1), dict(lda=3, K=4), dict(A=0), dict(x=0), dict(y=0),
    dict(A=GOOD + 2), dict(x=GOOD + 1), dict(y=GOOD + 2), dict(bias=GOOD + 1),
])
def test_f32_validation(args):
    a = dict(A=GOOD, lda=8, x=GOOD, bias=None, y=GOOD, M=4, K=8)
    a.update(args)
    rc = lg.gemv_f32(a["A"] or None, a["lda"], a["x"] or None, a["bias"],
                     a["y"] or None, a["M"], a["K"], None)
    assert rc == lg.GEMV_ERROR_INVALID_VALUE


@pytest.mark.parametrize("fn", [lg.gemv_f16, lg.gemv_bf16])
def test_half_validation(fn):
    assert fn(GOOD + 1, 8, GOOD, None, GOOD, 4, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
    assert fn(GOOD, 7, GOOD, None, GOOD, 4, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
    assert fn(None, 8, GOOD, None, GOOD, 4, 8, None) == lg.GEMV_ERROR_INVALID_VALUE


@pytest.mark.parametrize("fn", [lg.gemv_batched_f16, lg.gemv_batched_bf16])
@pytest.mark.parametrize("nvec", [0, 65, -3])
def test_batched_rejects_nvec(fn, nvec):
    assert fn(GOOD, 8, GOOD, None, GOOD, 4, 8, nvec, None) == lg.GEMV_ERROR_INVALID_VALUE


def test_empty_M_is_a_successful_no_op():
    # M == 0: nothing to compute and nothing enqueued
    assert lg.gemv_f32(None, 8, None, None, None, 0, 8, None) == lg.GEMV_SUCCESS
    assert lg.gemv_batched_bf16(None, 8, None, None, None, 0, 8, 4, None) == lg.GEMV_SUCCESS


def test_forced_family_must_fit_the_shape():
    r = lg.gemv_run_family(lg.DTYPE_F32, lg.FAMILY_BATCHED, GOOD, 8, GOOD, None,
                           GOOD, 4, 8, 2, None)
    assert r == lg.GEMV_ERROR_INVALID_VALUE
    r = lg.gemv_run_family(lg.DTYPE_F16, lg.FAMILY_WAVE_PER_ROW, GOOD, 8, GOOD,
                           None, GOOD, 4, 8, 2, None)
    assert r == lg.GEMV_ERROR_INVALID_VALUE
    with pytest.raises(lg.GemvError):
        lg.plan("f32", 4, 8, family=17)


# ---------------------------------------------------------------------------
# mapping table
# ---------------------------------------------------------------------------

ALIGNED = 1 << 20


def p(dtype, M, K, lda=None, nvec=1, A=ALIGNED, X=ALIGNED, family=lg.FAMILY_AUTO):
    return lg.plan(dtype, M, K, lda, nvec, A, X, family)


@pytest.mark.parametrize("dtype,K,lanes", [
    ("f32", 16, 4), ("f32", 32, 8), ("f32", 128, 32), ("f32", 4, 1),
    ("f32", 20, 8), ("bf16", 16, 2), ("bf16", 256, 32), ("f16", 64, 8),
    ("f32", 0, 1), ("f32", 3, 1),
])
def test_short_rows_share_a_wavefront(dtype, K, lanes):
    per16 = 4 if dtype == "f32" else 8
    lda = max(per16, -(-K // per16) * per16)  # 16-byte row pitch
    q = p(dtype, 1 << 20, K, lda=lda)
    assert q["family"] == lg.FAMILY_ROWS_PER_WAVE
    assert q["vector_loads"] == 1
    assert q["lanes_per_row"] == lanes
    assert q["rows_per_wave"] * q["lanes_per_row"] == 64
    # no lane idles beyond rounding the row's loads up to a power of two
    loads = -(-K // q["chunk_elems"])
    assert loads <= lanes < 2 * max(loads, 1) or lanes == 1
    assert q["grid"] * q["rows_per_group"] >= 1 << 20


def test_skinny_k16_geometry():
    q = p("f32", 1 << 20, 16)
    assert (q["lanes_per_row"], q["rows_per_wave"], q["row_tiles"]) == (4, 16, 4)
    assert q["rows_per_group"] == 16 * 4 * 4
    assert q["grid"] == (1 << 20) // q["rows_per_group"]


def test_row_tiles_of_tall_matrices():
    """At most 4 row tiles per wavefront; full 32-lane row groups take 2
    while that leaves 65536 workgroups, fewer rows keep 4, and problems
    below 1024 workgroups' worth keep one."""
    q = p("f32", 1 << 20, 128)  # 32 lanes per row, 2 rows per wavefront
    assert (q["lanes_per_row"], q["row_tiles"], q["grid"]) == (32, 2, 1 << 16)
    assert p("bf16", 1 << 20, 256)["row_tiles"] == 2
    assert p("f32", 1 << 18, 128)["row_tiles"] == 4
    assert p("f32", 1 << 20, 32)["row_tiles"] == 4
    assert p("f32", 1 << 22, 16)["row_tiles"] == 4
    assert p("f32", 1024 * 64, 16)["row_tiles"] == 1


def test_small_problem_spreads_out():
    q = p("f32", 1024, 128)  # the 1024 x 128 timing shape: launch-bound
    assert q["family"] == lg.FAMILY_ROWS_PER_WAVE and q["row_tiles"] == 1
    assert q["grid"] == 1024 // 8


def test_mid_rows_get_a_wavefront_each():
    q = p("bf16", 4096, 4096)
    assert q["family"] == lg.FAMILY_WAVE_PER_ROW
    assert q["lanes_per_row"] == 64 and q["rows_per_group"] == 4
    assert q["grid"] == 1024 and q["passes"] == 8 and q["batch"] == 8
    assert p("bf16", 1024, 4096)["family"] == lg.FAMILY_WAVE_PER_ROW


def test_wave_per_row_workgroups_balance_the_compute_units():
    """One row per wavefront: workgroups of 4 wavefronts, or of 2 when that
    leaves the busiest of the 256 compute units a smaller share of
    workgroups over the mean (384 workgroups of 4 put two on half the units
    and one on the rest; 768 of 2 put three on every unit)."""
    for M, waves in ((768, 4), (1024, 4), (1280, 2), (1535, 2), (1536, 2), (1537, 4), (1792, 4),
                     (2048, 4), (2304, 2), (2560, 2), (2816, 4), (3072, 4), (3584, 2), (4096, 4)):
        q = p("bf16", M, 4096)
        assert q["family"] == lg.FAMILY_WAVE_PER_ROW
        assert (q["waves_per_group"], q["block"], q["rows_per_group"]) == (waves, 64 * waves, waves), M
        assert q["grid"] == -(-M // waves)
    # the same for the forced family; element loads and short-row plans keep 4
    assert p("bf16", 1536, 4096, family=lg.FAMILY_WAVE_PER_ROW)["waves_per_group"] == 2
    assert p("bf16", 1536, 4096, A=ALIGNED + 2)["waves_per_group"] == 4
    assert p("f32", 1536, 2050)["waves_per_group"] == 2
    assert p("bf16", 1536, 256)["waves_per_group"] == 4  # rows per wavefront


def test_very_tall_short_rows_share_wavefronts():
    """With more than 16384 workgroups' worth of short rows, a wavefront
    takes 2, 4 or 8 rows (at most 8 loads per lane in flight); up to 65536
    such rows keep one row per wavefront."""
    q = p("f32", 1 << 20, 256)  # 64 loads: one per lane
    assert (q["family"], q["batch"], q["row_tiles"], q["grid"]) == \
        (lg.FAMILY_WAVE_PER_ROW, 1, 8, (1 << 20) // 32)
    q = p("bf16", 1 << 20, 1024)  # 128 loads: two per lane
    assert (q["batch"], q["row_tiles"], q["grid"]) == (2, 4, (1 << 20) // 16)
    assert p("bf16", 1 << 20, 1536)["row_tiles"] == 2  # three per lane
    assert p("bf16", 1 << 18, 4096)["row_tiles"] == 1 or p("bf16", 1 << 18, 4096)["family"] != \
        lg.FAMILY_WAVE_PER_ROW
    assert p("f32", 65536, 256)["row_tiles"] == 1
    assert p("f32", 65540, 256)["row_tiles"] == 2
    # element loads keep one row per wavefront
    assert p("f32", 1 << 20, 256, A=ALIGNED + 4)["row_tiles"] == 1


def test_wavefront_batches_fit_the_row():
    """A wavefront per row issues its row's loads in as few batches of at
    most 8 loads per lane as possible, all of one size."""
    for dtype, M, K, batch in (("bf16", 4096, 2048, 4), ("bf16", 4096, 1024, 2),
                               ("bf16", 4096, 3072, 6), ("bf16", 300, 5120, 5),
                               ("bf16", 300, 1000, 2), ("f32", 4096, 1024, 4),
                               ("bf16", 300, 8184, 8), ("bf16", 300, 7000, 7)):
        # (300 rows of 256 loads or more take a workgroup each automatically)
        q = p(dtype, M, K, family=lg.FAMILY_WAVE_PER_ROW if M == 300 else lg.FAMILY_AUTO)
        assert (q["family"], q["batch"]) == (lg.FAMILY_WAVE_PER_ROW, batch), (dtype, M, K)
        loads = -(-K // q["chunk_elems"])
        per_lane = -(-loads // 64)
        assert q["batch"] * -(-per_lane // q["batch"]) - per_lane < -(-per_lane // 8)


def test_long_or_many_rows_get_a_workgroup_each():
    q = p("bf16", 4096, 14336)  # 1792 loads per row: 7 per lane, one batch
    assert q["family"] == lg.FAMILY_GROUP_PER_ROW
    assert q["lanes_per_row"] == 256 and q["batch"] == 7 and q["passes"] == 7
    q = p("bf16", 14336, 4096)  # many rows of 512 loads: 2 per lane
    assert q["family"] == lg.FAMILY_GROUP_PER_ROW and q["batch"] == 2
    # "many" starts at 6144 rows (the fused q/k/v rows of one decode token)
    assert p("bf16", 6144, 4096)["family"] == lg.FAMILY_GROUP_PER_ROW
    assert p("bf16", 6143, 4096)["family"] == lg.FAMILY_WAVE_PER_ROW
    q = p("f32", 100, 1000)     # few rows: 250 loads, one per lane
    assert q["family"] == lg.FAMILY_GROUP_PER_ROW and q["batch"] == 1


def test_few_long_rows_get_a_workgroup_each():
    q = p("bf16", 256, 4096)
    assert q["family"] == lg.FAMILY_GROUP_PER_ROW
    assert q["grid"] == 256 and q["block"] == 256 and q["rows_per_group"] == 1
    # rows of at least 256 loads keep a workgroup each up to 704 rows
    for M in (257, 384, 512, 704):
        assert p("bf16", M, 4096)["family"] == lg.FAMILY_GROUP_PER_ROW, M
        assert p("bf16", M, 2048)["family"] == lg.FAMILY_GROUP_PER_ROW, M
    # shorter rows (some lanes of a workgroup would idle) and more rows: a
    # wavefront per row; 1024 rows already give every CU several wavefronts
    assert p("bf16", 512, 1024)["family"] == lg.FAMILY_WAVE_PER_ROW
    assert p("bf16", 705, 4096)["family"] == lg.FAMILY_WAVE_PER_ROW
    assert p("bf16", 1024, 4096)["family"] == lg.FAMILY_WAVE_PER_ROW


def test_worked_example_mapping():
    """Page "第 3 课：GEMV 与行级并行", section "具体演示与数值推演": M=3,
    N=1024 on 256 threads per row is 3 workgroups, each thread taking 4
    strided passes of one element.  The workgroup-per-row family with
    element loads (a misaligned A forces them) reproduces that geometry."""
    fx = json.loads((ROOT / "tests" / "golden" / "worked_example_m3_k1024.json").read_text())
    pg = fx["printed_by_the_page"]
    q = p("f32", pg["M"], pg["N"], A=ALIGNED + 4, family=lg.FAMILY_GROUP_PER_ROW)
    assert q["vector_loads"] == 0
    assert q["grid"] == pg["blocks"]
    assert q["lanes_per_row"] == pg["threads_per_block"] == q["block"]
    assert q["passes"] == pg["column_passes_per_row"]
    # with 16-byte loads the same row is one pass
    q = p("f32", pg["M"], pg["N"], family=lg.FAMILY_GROUP_PER_ROW)
    assert q["vector_loads"] == 1 and q["passes"] == 1


@pytest.mark.parametrize("kw", [dict(A=ALIGNED + 4), dict(X=ALIGNED + 8)])
def test_misaligned_falls_back_to_element_loads(kw):
    q = p("f32", 4096, 4096, **kw)
    assert q["vector_loads"] == 0 and q["chunk_elems"] == 1


def test_unaligned_rows_keep_16_byte_loads():
    """With aligned A and x, a row pitch or K that is not a whole number of
    16-byte loads still takes 16-byte loads for one vector (rows start at
    element-aligned addresses; the tail shorter than a load is read element
    by element); several vectors need the pitch aligned."""
    for dtype, M, K, lda in (("f32", 4096, 4096, 4097), ("bf16", 384, 43690, 43690),
                             ("f16", 4096, 4100, 4100), ("bf16", 6144, 2730, 2731)):
        q = p(dtype, M, K, lda=lda)
        assert q["vector_loads"] == 1 and q["chunk_elems"] == 16 // (4 if dtype == "f32" else 2)
    # several vectors on unaligned rows: the vector-ALU batched family, still
    # with 16-byte loads (the matrix cores need aligned operand rows)
    q = p("f16", 4096, 4100, nvec=4)
    assert q["family"] == lg.FAMILY_BATCHED and q["vector_loads"] == 1


def test_batched_plans():
    q = p("f16", 4096, 4096, nvec=16)
    assert q["family"] == lg.FAMILY_BATCHED_MFMA
    assert (q["rows_per_group"], q["waves_per_group"], q["grid"]) == (16, 8, 256)
    assert q["passes"] == 4096 // 64 // 8
    # the matrix cores need every 8-element group of a row aligned
    assert p("bf16", 4096, 4104, nvec=3)["family"] == lg.FAMILY_BATCHED_MFMA
    assert p("bf16", 4096, 4100, lda=4104, nvec=3)["family"] == lg.FAMILY_BATCHED
    assert p("bf16", 4096, 4096, nvec=3, A=ALIGNED + 2)["family"] == lg.FAMILY_BATCHED
    with pytest.raises(lg.GemvError):
        p("bf16", 4096, 4100, lda=4104, nvec=3, family=lg.FAMILY_BATCHED_MFMA)
    with pytest.raises(lg.GemvError):
        p("f32", 4096, 4096, nvec=1, family=lg.FAMILY_BATCHED_MFMA)
    q1 = p("f16", 4096, 4096, nvec=1)
    assert q1["family"] != lg.FAMILY_BATCHED   # nvec 1 is plain GEMV
    q = p("f16", 4096, 4095, nvec=4)  # X columns misaligned: unaligned 16-byte loads
    assert q["family"] == lg.FAMILY_BATCHED and q["vector_loads"] == 1
    with pytest.raises(lg.GemvError):
        p("f16", 4096, 4096, nvec=65)


def test_vector_alu_batched_rows_per_wavefront():
    """Two rows per wavefront once the 2-row grid (8 rows per workgroup)
    covers the 256 compute units twice, or more than once with 4 or more
    vectors; else one row, with twice as many workgroups."""
    for M, nvec, rows in ((1024, 2, 1), (2048, 16, 1), (2049, 3, 1), (2049, 4, 2),
                          (3072, 2, 1), (3072, 8, 2), (4088, 2, 1), (4089, 2, 2),
                          (4096, 16, 2), (8192, 5, 2), (7, 16, 1)):
        q = p("f16", M, 4100, nvec=nvec)
        assert q["family"] == lg.FAMILY_BATCHED, (M, nvec)
        assert q["rows_per_wave"] == rows, (M, nvec)
        # up to 512 rows the workgroup's 4 wavefronts share each row; up to
        # 1536 rows with 4 or more vectors, pairs of wavefronts
        split = 4 if M <= 512 else (2 if M <= 1536 and nvec >= 4 else 1)
        assert q["lanes_per_row"] == 64 * split, (M, nvec)
        per_group = rows * 4 // split
        assert q["rows_per_group"] == per_group and q["grid"] == -(-M // per_group), (M, nvec)
    # blocks of at most 16 vectors are planned one by one: 17 vectors on
    # 3000 rows run 16 on two rows per wavefront, then 1 on one
    assert p("bf16", 3000, 4100, nvec=17)["rows_per_wave"] == 2
    assert p("bf16", 3000, 4100, nvec=1, family=lg.FAMILY_BATCHED)["rows_per_wave"] == 1


def test_vector_alu_batched_k_split():
    """Up to 512 rows the vector-ALU batched kernel gives each row a whole
    workgroup (4 wavefronts, every fourth batch each, then an in-order fold
    of their totals: 3 more roundings); more rows keep a wavefront per row."""
    for M, K, nvec in ((1, 4100, 2), (7, 100, 16), (512, 11009, 16), (64, 14337, 5), (513, 4100, 3)):
        q = p("bf16", M, K, nvec=nvec)
        one = p("bf16", M, K, nvec=nvec, family=lg.FAMILY_BATCHED)
        assert q["family"] == lg.FAMILY_BATCHED and q == one
        if M <= 512:
            assert (q["lanes_per_row"], q["rows_per_wave"], q["rows_per_group"], q["grid"]) == \
                (256, 1, 1, M)
        else:
            assert (q["lanes_per_row"], q["rows_per_group"]) == (64, 4)
        assert q["waves_per_group"] == 4 and q["block"] == 256
        assert q["rounding_chain"] <= 150
    # the fold of 4 wavefronts' totals is charged to the bound
    split, whole = p("f16", 512, 4100, nvec=2), p("f16", 513, 4100, nvec=2)
    assert split["rounding_chain"] == whole["rounding_chain"] + 3
    # pairs of wavefronts per row: 513-1536 rows with at least 4 vectors
    for M, nvec, lanes in ((513, 4, 128), (600, 8, 128), (1536, 16, 128), (1536, 3, 64),
                           (1537, 8, 64), (1024, 2, 64)):
        q = p("f16", M, 4100, nvec=nvec)
        assert q["family"] == lg.FAMILY_BATCHED and q["lanes_per_row"] == lanes, (M, nvec, q)
        per_group = 4 * 64 // lanes
        assert (q["rows_per_group"], q["grid"]) == (per_group, -(-M // per_group)), (M, nvec)
    pair, one = p("f16", 1024, 4100, nvec=4), p("f16", 1537, 4100, nvec=4)
    assert pair["rounding_chain"] == one["rounding_chain"] + 1


def test_matrix_core_workgroup_shapes():
    """Up to 1024 rows a workgroup takes 4 rows (with X staged in LDS: more
    than 5 vectors), up to 2048 one group of 8 (each size fills the 256
    compute units at most once), else two groups of 8; more 16-row tiles
    than compute units: workgroups of 4 wavefronts (half the LDS, so two
    share a unit), each walking twice the 64-wide steps; otherwise 8."""
    for M, waves, groups, rows in ((16, 8, 1, 4), (1024, 8, 1, 4), (1025, 8, 1, 8), (2048, 8, 1, 8),
                                   (2049, 8, 2, 16), (4096, 8, 2, 16), (4097, 4, 2, 16),
                                   (6144, 4, 2, 16), (14336, 4, 2, 16)):
        for nvec in (3, 16, 33):
            want = 8 if nvec <= 5 and rows == 4 else rows  # X read straight from memory: 8
            q = p("f16", M, 4096, nvec=nvec)
            assert q["family"] == lg.FAMILY_BATCHED_MFMA
            if M == 14336 and nvec == 16:  # four groups (below)
                assert (q["row_tiles"], q["rows_per_group"], q["batch"]) == (4, 32, 4)
                continue
            assert (q["row_tiles"], q["rows_per_group"]) == (groups, want)
            assert (q["waves_per_group"], q["block"], q["grid"]) == \
                (waves, 64 * waves, -(-M // want))
            assert q["passes"] == 4096 // 64 // waves
            tiles = 1 if nvec <= 16 else (2 if nvec <= 32 else 4)
            assert q["lds_bytes"] == waves * 16 * tiles * (q["batch"] * 128 + 16) <= 20 * 1024 * waves
            assert q["rounding_chain"] <= 150


def test_matrix_core_four_row_groups():
    """6-16 vectors (X staged in LDS) on tall matrices: four groups of 8 rows
    (half the X bytes per A byte) when their grid has more workgroups than
    compute units and no unit runs more rows than with two groups (the
    largest number of workgroups on one unit times their rows)."""
    for M, nvec, groups in ((12288, 16, 2), (13312, 9, 4), (13312, 8, 4), (13313, 16, 4),
                            (14336, 16, 4), (14336, 6, 4), (16384, 12, 4), (20480, 16, 2),
                            (28672, 16, 2), (8192, 16, 2), (4096, 16, 2), (14336, 17, 2),
                            (14336, 5, 2)):
        q = p("f16", M, 4096, nvec=nvec)
        assert q["family"] == lg.FAMILY_BATCHED_MFMA
        g2, g4 = -(-M // 16), -(-M // 32)
        assert (groups == 4) == (6 <= nvec <= 16 and g4 > 256 and
                                 2 * -(-g4 // 256) <= -(-g2 // 256)), (M, nvec)
        assert q["row_tiles"] == groups and q["rows_per_group"] == 8 * groups, (M, nvec)
        if groups == 4:
            # half-size chunks, 4 wavefronts: 33 KiB of LDS, two workgroups per unit
            assert (q["waves_per_group"], q["batch"], q["grid"]) == (4, 4, g4)
            assert q["lds_bytes"] == 4 * 16 * (4 * 128 + 16)
            assert q["rounding_chain"] <= 150


def test_wide_batched_plans():
    """17-64 vectors: the matrix-core kernel takes 2 or 4 tiles of 16
    vectors per A operand, in chunks of 4 or 2 64-wide steps, so the X
    staged per chunk stays 16 KiB per wavefront and the LDS within 160 KiB;
    the vector-ALU family plans its first block of 16 vectors."""
    for nvec, chunk, tiles in ((16, 8, 1), (17, 4, 2), (32, 4, 2), (33, 2, 4), (64, 2, 4)):
        q = p("bf16", 4096, 4096, nvec=nvec)
        assert q["family"] == lg.FAMILY_BATCHED_MFMA and q["batch"] == chunk
        assert q["grid"] == 256 and q["block"] == 512
        assert q["lds_bytes"] == 8 * 16 * tiles * (chunk * 128 + 16) <= 160 * 1024
    for nvec in (17, 40, 64):
        wide = p("f16", 999, 1000, nvec=nvec, A=ALIGNED + 2)
        assert wide["column_blocks"] == -(-nvec // 16)
        assert {**wide, "column_blocks": 1} == p("f16", 999, 1000, nvec=16, A=ALIGNED + 2)


# ---------------------------------------------------------------------------
# fused entry points: validation without a GPU
# ---------------------------------------------------------------------------

def test_multi_validation():
    seg = (GOOD, 8, 4, None, GOOD)
    ok_table = lg.segment_table([seg, seg])
    for fn in (lg.gemv_multi_f32, lg.gemv_multi_f16, lg.gemv_multi_bf16):
        assert fn(ok_table, 0, GOOD, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        assert fn(ok_table, lg.MAX_SEGMENTS + 1, GOOD, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        assert fn(None, 1, GOOD, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        bad = lg.segment_table([seg, (GOOD, 7, 4, None, GOOD)])     # lda < K
        assert fn(bad, 2, GOOD, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        bad = lg.segment_table([seg, (None, 8, 4, None, GOOD)])     # NULL A
        assert fn(bad, 2, GOOD, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        bad = lg.segment_table([seg, (GOOD, 8, -1, None, GOOD)])    # M < 0
        assert fn(bad, 2, GOOD, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        empty = lg.segment_table([(None, 8, 0, None, None)] * 3)   # nothing to do
        assert fn(empty, 3, GOOD, 8, None) == lg.GEMV_SUCCESS


def test_gated_validation():
    for fn in (lg.gemv_gate_up_silu_f32, lg.gemv_gate_up_silu_f16, lg.gemv_gate_up_silu_bf16):
        assert fn(GOOD, GOOD, 7, GOOD, GOOD, 4, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        assert fn(None, GOOD, 8, GOOD, GOOD, 4, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        assert fn(GOOD, None, 8, GOOD, GOOD, 4, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        assert fn(GOOD, GOOD, 8, GOOD, None, 4, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        assert fn(GOOD, GOOD, 8, GOOD, GOOD, -1, 8, None) == lg.GEMV_ERROR_INVALID_VALUE
        assert fn(None, None, 8, None, None, 0, 8, None) == lg.GEMV_SUCCESS


def test_gated_family_is_not_a_plain_gemv():
    assert lg.gemv_run_family(lg.DTYPE_BF16, lg.FAMILY_GATED_SILU, GOOD, 8, GOOD, None,
                              GOOD, 4, 8, 1, None) == lg.GEMV_ERROR_INVALID_VALUE


# ---------------------------------------------------------------------------
# split-K: validation, workspace size and slice geometry, without a GPU
# ---------------------------------------------------------------------------

SPLITK = (lg.gemv_splitk_f32, lg.gemv_splitk_f16, lg.gemv_splitk_bf16)


def test_splitk_validation():
    big_K = 1 << 20            # 4 rows of 2^20: the automatic plan splits
    for fn in SPLITK:
        def call(M=4, K=big_K, lda=big_K, splits=0, ws=GOOD, ws_bytes=1 << 20, y=GOOD):
            return fn(GOOD, lda, GOOD, None, y, M, K, splits, ws, ws_bytes, None)
        assert call(splits=-1) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(lda=big_K - 1) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(M=-1) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(y=None) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(ws=None) == lg.GEMV_ERROR_INVALID_VALUE          # needed, missing
        assert call(ws=GOOD + 2) == lg.GEMV_ERROR_INVALID_VALUE      # misaligned
        assert call(ws_bytes=16) == lg.GEMV_ERROR_INVALID_VALUE      # too small
        assert call(M=0, ws=None, ws_bytes=0) == lg.GEMV_SUCCESS     # nothing to do


def test_splitk_family_is_not_a_plain_gemv():
    assert lg.gemv_run_family(lg.DTYPE_F32, lg.FAMILY_SPLIT_K, GOOD, 8, GOOD, None,
                              GOOD, 4, 8, 1, None) == lg.GEMV_ERROR_INVALID_VALUE
    with pytest.raises(lg.GemvError):
        lg.plan("f32", 4, 8, family=lg.FAMILY_SPLIT_K)


def test_splitk_workspace_size():
    n = ctypes.c_size_t(7)
    assert lg.gemv_splitk_workspace_size(0, 4, 8, -1, ctypes.byref(n)) == lg.GEMV_ERROR_INVALID_VALUE
    assert lg.gemv_splitk_workspace_size(0, -1, 8, 0, ctypes.byref(n)) == lg.GEMV_ERROR_INVALID_VALUE
    assert lg.gemv_splitk_workspace_size(3, 4, 8, 0, ctypes.byref(n)) == lg.GEMV_ERROR_INVALID_VALUE
    assert lg.gemv_splitk_workspace_size(0, 4, 8, 0, None) == lg.GEMV_ERROR_INVALID_VALUE
    # rows too short or numerous enough: no split, no workspace
    assert lg.splitk_workspace_size("bf16", 4096, 4096) == 0
    assert lg.splitk_workspace_size("f32", 16, 1000) == 0
    p = lg.plan_splitk("f32", 16, 1 << 20)
    assert lg.splitk_workspace_size("f32", 16, 1 << 20) == 4 * 16 * p["splits"]


def test_splitk_for_few_long_rows():
    """The small-M case: fewer than 192 rows of at least 8192 16-byte loads
    are cut into slices so that rows × slices approaches 1024 workgroups, each
    slice at least 512 loads and a whole number of 64-lane loads, and the
    slice count a multiple of the 8 XCDs once it reaches 8; a workgroup takes
    two rows of a slice (one when M = 1), so that each x chunk serves both."""
    for dtype, M, K in (("f32", 16, 1 << 20), ("f32", 8, 1 << 21), ("bf16", 64, 1 << 18),
                        ("f16", 1, 1 << 24), ("bf16", 100, 100000), ("f32", 191, 1 << 15),
                        ("bf16", 32, 65536)):
        p = lg.plan_splitk(dtype, M, K, A_addr=ALIGNED, x_addr=ALIGNED)
        s = 4 if dtype == "f32" else 2
        assert p["family"] == lg.FAMILY_SPLIT_K, (dtype, M, K)
        assert p["splits"] >= 2 and M * p["splits"] <= 1024
        assert (p["slice_elems"] * s) % 16 == 0
        assert p["slice_elems"] * s >= 512 * 16 and (p["slice_elems"] * s // 16) % 64 == 0
        assert (p["splits"] - 1) * p["slice_elems"] < K <= p["splits"] * p["slice_elems"]
        assert p["splits"] < 8 or p["splits"] % 8 == 0
        U = 2 if M >= 2 else 1
        assert p["rows_per_group"] == U
        assert p["grid"] == -(-M // U) * p["splits"] and p["block"] == 256
        per_lane = -(-p["slice_elems"] * s // 16 // 256)
        assert p["batch"] == -(-per_lane // -(-per_lane // 8))  # equal batches of <= 8


def test_splitk_keeps_the_plain_plan_when_it_fills_the_gpu():
    for dtype, M, K in (("bf16", 4096, 4096), ("bf16", 1024, 4096), ("bf16", 1000, 40000),
                        ("f32", 16, 1000), ("f32", 1 << 20, 16), ("bf16", 5, 0),
                        ("bf16", 256, 1 << 16), ("bf16", 512, 1 << 15), ("bf16", 64, 14336),
                        ("bf16", 192, 1 << 16), ("f32", 255, 1 << 15),
                        ("f32", 100, 32764)):           # 8191 loads per row
        p = lg.plan_splitk(dtype, M, K, A_addr=ALIGNED, x_addr=ALIGNED)
        assert p["splits"] == 1 and p["slice_elems"] == K
        assert p == {**lg.plan(dtype, M, K, A_addr=ALIGNED, X_addr=ALIGNED),
                     "splits": 1, "slice_elems": K}


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_splitk_requested_slices(dtype):
    s = 4 if dtype == "f32" else 2
    g = 16 // s
    for M, K, want in ((7, 1000, 3), (3, 10, 100), (2, 1 << 20, 5000), (1, 8, 2), (4, 129, 2),
                       (9, 4097, 7), (1, 1, 3)):
        p = lg.plan_splitk(dtype, M, K, splits=want, A_addr=ALIGNED, x_addr=ALIGNED)
        S, sl = p["splits"], p["slice_elems"]
        assert 1 <= S <= min(want, 1024)
        assert (S - 1) * sl < K <= S * sl or (K == 0 and S == 1)
        if S > 1:
            assert sl % g == 0 and p["family"] == lg.FAMILY_SPLIT_K
    assert lg.plan_splitk(dtype, 7, 1000, splits=3)["slice_elems"] == -(-(-(-1000 // 3)) // g) * g


def test_splitk_geometry_properties():
    """Over many shapes: slices cover K exactly once, automatic counts of 8 or
    more are multiples of 8, and the workspace matches rows × slices."""
    import random
    rnd = random.Random(7)
    for _ in range(3000):
        dtype = rnd.choice(["f32", "f16", "bf16"])
        M = rnd.choice([0, 1, 2, 3, 7, 8, 31, 64, 100, 255, 256, 1000, rnd.randint(1, 300)])
        K = rnd.choice([0, 1, 15, 4096, 8192 * 8, rnd.randint(1, 1 << 22), rnd.randint(1 << 16, 1 << 24)])
        splits = rnd.choice([0, 0, 0, 1, 2, 3, 8, 100, 5000])
        p = lg.plan_splitk(dtype, M, K, splits=splits, A_addr=ALIGNED, x_addr=ALIGNED)
        S, sl = p["splits"], p["slice_elems"]
        assert S >= 1 and S <= 1024
        if S == 1:
            assert sl == K and p["family"] != lg.FAMILY_SPLIT_K
            assert lg.splitk_workspace_size(dtype, M, K, splits) == 0
            continue
        assert p["family"] == lg.FAMILY_SPLIT_K
        assert (S - 1) * sl < K <= S * sl
        assert (sl * (4 if dtype == "f32" else 2)) % 16 == 0
        if splits == 0:
            assert M < 192 and (S < 8 or S % 8 == 0) and M * S <= 1024
        else:
            assert S <= splits
        assert lg.splitk_workspace_size(dtype, M, K, splits) == 4 * M * S


# ---------------------------------------------------------------------------
# weight-only int8: validation and mapping, without a GPU
# ---------------------------------------------------------------------------

Q8 = (lg.gemv_q8_f32, lg.gemv_q8_f16, lg.gemv_q8_bf16)


def test_q8_validation():
    for fn, s in zip(Q8, (4, 2, 2)):
        def call(Q=GOOD, ldq=64, scale=GOOD, x=GOOD, bias=None, y=GOOD, M=4, K=64):
            return fn(Q, ldq, scale, x, bias, y, M, K, None)
        assert call(M=-1) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(K=-1) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(ldq=63) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(Q=None) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(x=None) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(y=None) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(scale=None) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(scale=GOOD + 2) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(bias=GOOD + 1) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(y=GOOD + 2) == lg.GEMV_ERROR_INVALID_VALUE
        assert call(x=GOOD + s - 1) == lg.GEMV_ERROR_INVALID_VALUE   # x not element-aligned
        assert call(M=0, Q=None, x=None, y=None, scale=None) == lg.GEMV_SUCCESS
    # the x type code must be a float type
    assert lg.gemv_q8_run_family(3, lg.FAMILY_AUTO, GOOD, 64, GOOD, GOOD, None, GOOD, 4, 64,
                                 None) == lg.GEMV_ERROR_INVALID_VALUE


def test_q8_x_in_registers():
    """int8 rows whose x is longer than 8 KiB and fits 4 chunks per lane of
    4 wavefronts (3 with fp32 x), K a whole number of 16-weight loads, and
    enough rows for 256 workgroups of 2 or 4: x is loaded once per workgroup
    and kept in registers while it walks its rows."""
    for xd, M, K, rows, chunks in (("f16", 4096, 11008, 4, 3), ("bf16", 4096, 11008, 4, 3),
                                   ("f16", 1024, 16384, 4, 4), ("f32", 4096, 8192, 4, 2),
                                   ("f32", 4096, 12288, 4, 3), ("f16", 700, 11008, 2, 3)):
        p = lg.plan_q8(xd, M, K, Q_addr=ALIGNED, x_addr=ALIGNED)
        assert (p["family"], p["x_in_registers"], p["row_tiles"], p["batch"]) == \
            (lg.FAMILY_GROUP_PER_ROW, 1, rows, chunks), (xd, M, K, p)
        assert (p["waves_per_group"], p["lanes_per_row"], p["grid"]) == (4, 256, -(-M // rows))
        assert p["rounding_chain"] <= 150
    for xd, M, K in (("f16", 4096, 4096),     # an 8 KiB x: no
                     ("f16", 4096, 16400),    # 5 chunks per lane
                     ("f32", 4096, 12304),    # fp32 x, 4 chunks per lane
                     ("f16", 4096, 11000),    # not whole 16-weight loads
                     ("f16", 300, 11008)):    # too few rows for 256 workgroups of 2
        p = lg.plan_q8(xd, M, K, Q_addr=ALIGNED, x_addr=ALIGNED)
        assert p["x_in_registers"] == 0, (xd, M, K, p)
    # element loads never keep x in registers
    assert lg.plan_q8("f16", 4096, 11008, Q_addr=ALIGNED + 1, x_addr=ALIGNED)["x_in_registers"] == 0


def test_q8_families():
    """int8 weights run the three single-vector row families only, planned by
    their 1-byte rows: 16 weights per 16-byte load."""
    for fam in (lg.FAMILY_BATCHED, lg.FAMILY_BATCHED_MFMA, lg.FAMILY_SPLIT_K):
        with pytest.raises(lg.GemvError):
            lg.plan_q8("f16", 64, 4096, family=fam, Q_addr=ALIGNED, x_addr=ALIGNED)
    # K = 16 int8 weights are one load: one lane per row, 64 rows per wavefront
    p = lg.plan_q8("f16", 1000, 16, Q_addr=ALIGNED, x_addr=ALIGNED)
    assert (p["family"], p["lanes_per_row"], p["rows_per_wave"]) == (lg.FAMILY_ROWS_PER_WAVE, 1, 64)
    assert p["chunk_elems"] == 16
    # 4096 weights are 256 loads: a workgroup per row up to 4096 rows, a
    # workgroup per two rows up to 16384 rows (or from a 16 KiB x row on);
    # past that a wavefront per row, 4 loads per lane in flight, two rows per
    # wavefront once there are workgroups enough
    p = lg.plan_q8("bf16", 4096, 4096, Q_addr=ALIGNED, x_addr=ALIGNED)
    assert (p["family"], p["batch"], p["row_tiles"], p["grid"]) == \
        (lg.FAMILY_GROUP_PER_ROW, 2, 1, 4096)
    # (a row of at most two loads per lane of two wavefronts: two wavefronts)
    assert (p["waves_per_group"], p["lanes_per_row"], p["lds_bytes"]) == (2, 128, 8)
    # a 16 KiB fp32 x row: x in registers across 4 rows (one chunk per lane)
    p = lg.plan_q8("f32", 4096, 4096, Q_addr=ALIGNED, x_addr=ALIGNED)
    assert (p["family"], p["x_in_registers"], p["row_tiles"], p["batch"], p["grid"]) == \
        (lg.FAMILY_GROUP_PER_ROW, 1, 4, 1, 1024)
    p = lg.plan_q8("bf16", 14336, 4096, Q_addr=ALIGNED, x_addr=ALIGNED)
    assert (p["family"], p["batch"], p["row_tiles"], p["grid"]) == \
        (lg.FAMILY_GROUP_PER_ROW, 1, 2, 7168)
    assert p["lds_bytes"] == 4 * 2 * 4
    p = lg.plan_q8("bf16", 16384, 4096, Q_addr=ALIGNED, x_addr=ALIGNED)
    assert (p["family"], p["row_tiles"], p["grid"]) == (lg.FAMILY_GROUP_PER_ROW, 2, 8192)
    p = lg.plan_q8("bf16", 16392, 4096, Q_addr=ALIGNED, x_addr=ALIGNED)
    assert (p["family"], p["batch"], p["row_tiles"]) == (lg.FAMILY_WAVE_PER_ROW, 4, 2)
    assert p["grid"] == 16392 // 8
    # element loads keep one row per workgroup
    p = lg.plan_q8("f32", 4096, 4096, Q_addr=ALIGNED + 1, x_addr=ALIGNED)
    assert (p["family"], p["row_tiles"], p["vector_loads"]) == (lg.FAMILY_GROUP_PER_ROW, 1, 0)
    assert lg.plan_q8("bf16", 4096, 2048, Q_addr=ALIGNED, x_addr=ALIGNED)["family"] == \
        lg.FAMILY_WAVE_PER_ROW  # 128 loads: half a workgroup's lanes would idle
    p = lg.plan_q8("bf16", 300, 4096, family=lg.FAMILY_WAVE_PER_ROW, Q_addr=ALIGNED,
                   x_addr=ALIGNED)
    assert p["row_tiles"] == 1 and p["grid"] == 75
    # few, long rows: a workgroup per row, batches capped at 4
    p = lg.plan_q8("bf16", 100, 100000, Q_addr=ALIGNED, x_addr=ALIGNED)
    assert (p["family"], p["batch"], p["grid"]) == (lg.FAMILY_GROUP_PER_ROW, 4, 100)
    # byte-aligned Q or an odd row pitch fall back to element loads
    assert lg.plan_q8("f16", 64, 4096, Q_addr=ALIGNED + 1, x_addr=ALIGNED)["vector_loads"] == 0
    # an unaligned row pitch keeps 16-byte loads (rows start anywhere)
    assert lg.plan_q8("f16", 64, 4096, ldq=4100, Q_addr=ALIGNED, x_addr=ALIGNED)["vector_loads"] == 1


def test_long_x_rows_share_a_workgroup():
    """An x longer than 8 KiB and at most 6 chunks per lane of a 4-wavefront
    workgroup (bf16 4096 < K <= 12288, fp32 2048 < K <= 6144, K whole chunks)
    stays in registers while the workgroup walks 4 rows (2 when 4 would leave
    fewer than 256 workgroups), also for shapes a wavefront per row would
    otherwise run.  Longer x, or K not whole chunks, runs two rows per
    workgroup sharing each x chunk once x is longer than 16 KiB.  Shorter x
    keeps one row per workgroup."""
    q = p("bf16", 4096, 12288)
    assert (q["family"], q["row_tiles"], q["rows_per_group"], q["grid"], q["x_in_registers"]) == \
        (lg.FAMILY_GROUP_PER_ROW, 4, 4, 1024, 1)
    assert (q["batch"], q["block"], q["lds_bytes"]) == (6, 256, 64)
    q = p("bf16", 1000, 12288)
    assert (q["row_tiles"], q["grid"], q["x_in_registers"]) == (2, 500, 1)
    assert p("bf16", 300, 12288)["grid"] == 300
    # 8 KiB < x <= 16 KiB: rows a wavefront per row would run keep x in registers too
    for dtype, M, K, chunks in (("bf16", 4096, 6144, 3), ("bf16", 4096, 8192, 4),
                                ("f16", 2048, 4104, 3), ("f32", 4096, 2052, 3)):
        q = p(dtype, M, K)
        assert (q["family"], q["x_in_registers"], q["batch"], q["row_tiles"]) == \
            (lg.FAMILY_GROUP_PER_ROW, 1, chunks, 4), (dtype, M, K)
    # too few rows for two per workgroup: one row per workgroup (x from the caches)
    q = p("bf16", 500, 6144)
    assert q["family"] == lg.FAMILY_GROUP_PER_ROW and q["x_in_registers"] == 0
    q = p("bf16", 800, 6144)  # 400 pairs of rows: x in registers, two rows per workgroup
    assert q["x_in_registers"] == 1 and q["row_tiles"] == 2
    assert p("bf16", 4096, 4096)["family"] == lg.FAMILY_WAVE_PER_ROW
    assert p("f32", 2051, 6144)["batch"] == 6 and p("f32", 1025, 4100)["batch"] == 5
    # 7 chunks per lane (bf16 4096 x 14336: two rows per workgroup measured
    # faster), x past 24 KiB, or K not whole chunks: two rows share each x chunk
    for dtype, M, K, batch in (("bf16", 4096, 14336, 7), ("bf16", 4096, 14344, 8),
                               ("bf16", 4096, 14340, 7), ("f32", 4096, 8192, 8),
                               ("f32", 2051, 7168, 7)):
        q = p(dtype, M, K)
        assert (q["row_tiles"], q["batch"], q["x_in_registers"]) == (2, batch, 0), (dtype, K)
    assert p("bf16", 1000, 14336)["grid"] == 500
    # element loads never keep x in registers
    q = p("bf16", 4096, 12288, A=ALIGNED + 2)
    assert q["vector_loads"] == 0 and q["x_in_registers"] == 0
    assert p("f32", 515, 8300, family=lg.FAMILY_GROUP_PER_ROW)["grid"] == 258
    for dtype, M, K in (("bf16", 14336, 4096), ("bf16", 510, 8192), ("bf16", 100, 100000),
                        ("bf16", 510, 50000)):
        q = p(dtype, M, K, family=lg.FAMILY_GROUP_PER_ROW)
        assert q["row_tiles"] == 1 and q["grid"] == M
    # the loads of both rows' batch stay within 16 per lane
    for K in (4104, 8200, 12288, 14336, 14344, 30000, 1 << 20):
        q = p("bf16", 4096, K, family=lg.FAMILY_GROUP_PER_ROW)
        assert q["x_in_registers"] or q["row_tiles"] * q["batch"] <= 16
        # with x in registers: the row's chunks and the next row's in flight
        assert not q["x_in_registers"] or 3 <= q["batch"] <= 6


def test_read_probe_validation():
    sink = GOOD
    assert lg.gemv_read_probe(GOOD, 0, None, None) == lg.GEMV_SUCCESS  # nothing to read
    for buf, n, snk in ((None, 1024, sink), (GOOD, 1024, None), (GOOD, 1000, sink),
                        (GOOD + 8, 1024, sink), (GOOD, 1024, sink + 2)):
        assert lg.gemv_read_probe(buf, n, snk, None) == lg.GEMV_ERROR_INVALID_VALUE


def test_few_long_rows_take_wider_workgroups():
    """Below 1024 rows, rows that need more than one batch of loads per lane
    of 4 wavefronts get wider workgroups: 16 wavefronts for one row, 8 for a
    pair of rows sharing x; shorter rows, taller matrices and x held in
    registers keep 4."""
    def plan(dtype, M, K):
        return lg.plan(dtype, M, K, A_addr=ALIGNED, X_addr=ALIGNED)
    for dtype, M, K, waves, rows in (("bf16", 192, 65536, 16, 1), ("f32", 256, 32768, 16, 1),
                                     ("bf16", 384, 32768, 16, 1), ("bf16", 512, 32768, 8, 2),
                                     ("f16", 1000, 20000, 8, 2), ("bf16", 1023, 20000, 8, 2),
                                     ("bf16", 1024, 20000, 4, 2), ("bf16", 768, 16384, 4, 2),
                                     ("bf16", 256, 4096, 4, 1), ("bf16", 4096, 14336, 4, 2),
                                     ("bf16", 600, 8192, 4, 2)):   # x in registers
        p = plan(dtype, M, K)
        assert p["family"] == lg.FAMILY_GROUP_PER_ROW, (dtype, M, K)
        assert (p["waves_per_group"], p["row_tiles"]) == (waves, rows), (dtype, M, K, p)
        assert p["block"] == 64 * waves and p["lanes_per_row"] == 64 * waves
        assert p["grid"] == -(-M // rows) and p["lds_bytes"] == 4 * waves * rows
        s = 4 if dtype == "f32" else 2
        per_lane = -(-(K * s // 16) // (64 * waves))
        assert p["batch"] == -(-per_lane // -(-per_lane // 8))  # equal batches of <= 8
    assert plan("bf16", 600, 8192)["x_in_registers"] == 1
    # int8 weights keep 4 wavefronts
    q = lg.plan_q8("bf16", 256, 65536, Q_addr=ALIGNED, x_addr=ALIGNED)
    assert q["family"] == lg.FAMILY_GROUP_PER_ROW and q["waves_per_group"] == 4


def test_very_tall_rows_of_odd_load_counts_split_their_lanes():
    """Rows of 3-32 loads that are not a power of two: a very tall matrix
    (a grid of at least 16384 workgroups) gives each row 8 or 16 lanes with
    several loads each when that leaves fewer lanes idle; shorter matrices and
    power-of-two rows keep one load per lane."""
    for dtype, M, K, lanes, batch in (("f32", 1 << 20, 80, 8, 3), ("f32", 1 << 20, 96, 8, 3),
                                      ("bf16", 1 << 20, 160, 8, 3), ("f16", 530001, 176, 8, 3)):
        q = p(dtype, M, K)
        assert (q["family"], q["lanes_per_row"], q["batch"], q["row_tiles"]) == \
            (lg.FAMILY_ROWS_PER_WAVE, lanes, batch, 1), (dtype, M, K)
        assert q["grid"] == -(-M // (64 // lanes * 4)) >= 16384
    for dtype, M, K in (("f32", 1 << 18, 80), ("f32", 1 << 20, 40), ("f32", 1 << 20, 64),
                        ("f32", 1 << 20, 112)):
        assert p(dtype, M, K)["batch"] == 1, (dtype, M, K)


def test_read_probe_variant_validation():
    """The read-pattern probe takes 2/4/8/16 loads per lane, 1/2/4/8/16
    wavefronts per workgroup, at least one block per wavefront, flags in
    bits 0-2, and a timestamp buffer of 2 entries per wavefront."""
    f = lg.gemv_read_probe_variant
    ok = dict(buf=GOOD, n=1 << 20, sink=GOOD, loads=8, waves=4, blocks=1, flags=0,
              times=None, tlen=0)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["buf"], a["n"], a["sink"], a["loads"], a["waves"], a["blocks"], a["flags"],
                 a["times"], a["tlen"], None)
    assert call(n=0, buf=None) == lg.GEMV_SUCCESS  # nothing to read
    for bad in (dict(loads=3), dict(loads=32), dict(waves=3), dict(waves=32), dict(blocks=0),
                dict(flags=8), dict(buf=None), dict(sink=None), dict(n=1000), dict(buf=GOOD + 8),
                dict(times=GOOD + 4, tlen=1 << 20)):
        assert call(**bad) == lg.GEMV_ERROR_INVALID_VALUE, bad
    # 1 MiB with 8 KiB per wavefront: 128 wavefronts, 256 timestamps needed
    assert call(times=GOOD, tlen=255) == lg.GEMV_ERROR_INVALID_VALUE
