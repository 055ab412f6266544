"""Host-side properties of the planner that no GPU is needed for: the
matrix-core kernel's step partition, a compiled kernel behind every
automatic plan, and the rounding-chain bound of every plan."""

import ctypes
import math
import shutil
import subprocess
from pathlib import Path

import numpy as np
import pytest

import memory_bound_gemv_f32_amd as lg

TESTS = Path(__file__).resolve().parent
ALIGNED = 1 << 20
WAVES = (8, 4)  # wavefronts of a matrix-core workgroup (4 past one tile per compute unit)


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    out = tmp_path_factory.mktemp("shim") / "libplan_shim.so"
    subprocess.run([gxx, "-std=c++17", "-O1", "-shared", "-fPIC", str(TESTS / "plan_shim.cpp"),
                    "-o", str(out)], check=True)
    lib = ctypes.CDLL(str(out))
    lib.shim_mfma_step_range.argtypes = [ctypes.c_int] * 3 + [ctypes.POINTER(ctypes.c_int)] * 2
    lib.shim_compensated_roundings.argtypes = [ctypes.c_longlong]
    return lib


def step_range(lib, K, wave, waves):
    f, e = ctypes.c_int(), ctypes.c_int()
    lib.shim_mfma_step_range(K, waves, wave, ctypes.byref(f), ctypes.byref(e))
    return f.value, e.value


def groups_covered(lib, K, ch, waves):
    """How often the matrix-core kernel's loops visit each 8-element group of
    a row: whole chunks of `ch` 64-element steps, then the rest of the run
    one step at a time, reading only groups that start below K."""
    n_groups = K // 8
    seen = np.zeros(n_groups + 16, dtype=np.int64)
    whole = K // 64
    for wave in range(waves):
        first, end = step_range(lib, K, wave, waves)
        c = first
        s1 = min(end, whole)
        while c + ch <= s1:
            seen[8 * c: 8 * (c + ch)] += 1
            c += ch
        while c < end:
            lo, hi = 8 * c, min(8 * c + 8, n_groups)
            seen[lo:hi] += 1
            c += 1
    return seen[:n_groups], seen[n_groups:]


def test_mfma_steps_cover_every_group_once(shim):
    """Every K % 8 == 0 up to 2^16 (the lengths the matrix-core kernel
    takes), for the chunk lengths of 1, 2 and 4 vector tiles: each 8-element
    group of a row is visited exactly once, nothing past K is, the partial
    last step included (the K = 72..120, 136..184, ... lengths that lost it)."""
    for waves in WAVES:
        for ch in (8, 4, 2):
            for K in range(8, (1 << 16) + 1, 8):
                inside, past = groups_covered(shim, K, ch, waves)
                assert np.all(inside == 1), (K, ch, waves, np.flatnonzero(inside != 1)[:5])
                assert not past.any(), (K, ch, waves)


def test_mfma_step_runs_are_contiguous(shim):
    for waves in WAVES:
        for K in (0, 8, 64, 72, 200, 4096, 4104, 2680, 65536, 1 << 20):
            steps = -(-K // 64)
            runs = [step_range(shim, K, w, waves) for w in range(waves)]
            assert runs[0][0] == 0 and runs[-1][1] == steps
            for (f0, e0), (f1, e1) in zip(runs, runs[1:]):
                assert f0 <= e0 == f1 <= e1


def test_compensated_roundings(shim):
    assert shim.shim_compensated_roundings(1) == 0
    assert shim.shim_compensated_roundings(2) == 1
    assert shim.shim_compensated_roundings(4096) == 2
    # about one more rounding per (2^12)^2 / 2^24 ... grows only quadratically slowly
    assert shim.shim_compensated_roundings(1 << 17) <= 1100


# ---------------------------------------------------------------------------
# a compiled kernel behind every automatic plan
# ---------------------------------------------------------------------------

ROW_COUNTS = [1, 2, 3, 7, 64, 191, 192, 255, 256, 257, 511, 1000, 1023, 1024, 4096, 6143, 6144,
              14336, 65536, 65540, 262147, 524288, 524301, 1 << 20]
ROW_BYTES = [0, 2, 16, 48, 64, 80, 96, 128, 160, 176, 256, 260, 320, 368, 384, 512, 520, 1024,
             2048, 4096, 8192, 8208, 12288, 16384, 16400, 24576, 24592, 28672, 32768, 65536,
             1 << 18, 1 << 21]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_every_automatic_plan_has_a_kernel(dtype):
    """gemv_plan answers only for plans the entry points can launch (it checks
    that a compiled kernel exists): every shape, pitch and alignment below
    gets one."""
    es = {"f32": 4, "f16": 2, "bf16": 2}[dtype]
    for M in ROW_COUNTS:
        for rb in ROW_BYTES:
            K = rb // es
            for lda, A in ((K, ALIGNED), (K + 1, ALIGNED), (K, ALIGNED + es)):
                lg.plan(dtype, M, K, lda, 1, A, A)
                if dtype != "f32":
                    for nvec in (2, 5, 16, 17, 40, 64):
                        if M * K <= 1 << 28:
                            lg.plan(dtype, M, K, lda, nvec, A, A)


def _launchable(q, M):
    """What every plan must satisfy to be launched as planned: whole
    wavefronts, at most 1024 threads and 160 KiB of LDS per workgroup, and a
    grid whose workgroups cover the rows exactly (the last one possibly
    partly past the end)."""
    assert q["block"] % 64 == 0 and 64 <= q["block"] <= 1024, q
    assert q["block"] == 64 * q["waves_per_group"], q
    assert 0 <= q["lds_bytes"] <= 160 * 1024, q
    rows = q["rows_per_group"]
    tiles = q["grid"] // q["splits"] if q["family"] == lg.FAMILY_SPLIT_K else q["grid"]
    assert rows >= 1 and (tiles - 1) * rows < M <= tiles * rows, (M, q)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_every_plan_is_launchable(dtype):
    checked = 0
    es = {"f32": 4, "f16": 2, "bf16": 2}[dtype]
    for M in ROW_COUNTS + [1025, 1535, 1536, 2048, 2049, 2560, 4097, 4113]:
        for rb in ROW_BYTES:
            K = rb // es
            if K == 0 or M * K > 1 << 34:
                continue
            for lda, A in ((K, ALIGNED), (K + 1, ALIGNED), (K, ALIGNED + es)):
                for fam in (lg.FAMILY_AUTO, lg.FAMILY_ROWS_PER_WAVE, lg.FAMILY_WAVE_PER_ROW,
                            lg.FAMILY_GROUP_PER_ROW):
                    try:
                        q = lg.plan(dtype, M, K, lda, 1, A, A, fam)
                    except lg.GemvError:
                        continue
                    _launchable(q, M)
                    checked += 1
                if dtype != "f32":
                    for nvec in (2, 5, 6, 16, 33, 64):
                        if M * K * nvec > 1 << 34:
                            continue
                        for fam in (lg.FAMILY_AUTO, lg.FAMILY_BATCHED, lg.FAMILY_BATCHED_MFMA):
                            try:
                                q = lg.plan(dtype, M, K, lda, nvec, A, A, fam)
                            except lg.GemvError:
                                continue
                            _launchable(q, M)
                            checked += 1
            if M < 192 and K >= 8192:
                q = lg.plan_splitk(dtype, M, K, A_addr=ALIGNED, x_addr=ALIGNED)
                _launchable(q, M)
    assert checked > 1000


@pytest.mark.parametrize("xdtype", ["f32", "f16", "bf16"])
def test_every_automatic_int8_plan_has_a_kernel(xdtype):
    """Int8 rows of 17-24 loads on very tall matrices (K 257..384 at 2^19 rows
    and more) had a plan with no kernel behind it; now every shape has one."""
    for M in ROW_COUNTS:
        # (4112-16384: x kept in registers over 2-4 rows, 1-4 chunks per lane,
        # 16400 just past it; with fp32 x 12288 is the last)
        for K in [0, 1, 16, 17, 48, 100, 256, 257, 272, 320, 368, 384, 385, 512, 1000, 4096,
                  4112, 8192, 8320, 11008, 12288, 12304, 14336, 16384, 16400, 100000]:
            for ldq, Q in ((K, ALIGNED), (K + 3, ALIGNED), (K, ALIGNED + 1)):
                q = lg.plan_q8(xdtype, M, K, ldq, Q, ALIGNED)
                assert q["batch"] == 1 or q["lanes_per_row"] == 64 or \
                    q["family"] == lg.FAMILY_GROUP_PER_ROW, (M, K, q)
                if K > 0:
                    _launchable(q, M)


def test_tall_int8_rows_keep_one_load_per_lane():
    for M, K in ((524288, 320), (524288, 368), (1 << 20, 320)):
        q = lg.plan_q8("bf16", M, K, K, ALIGNED, ALIGNED)
        assert q["family"] == lg.FAMILY_ROWS_PER_WAVE and q["batch"] == 1, q


# ---------------------------------------------------------------------------
# the rounding-chain bound
# ---------------------------------------------------------------------------

FAMILIES = [lg.FAMILY_AUTO, lg.FAMILY_ROWS_PER_WAVE, lg.FAMILY_WAVE_PER_ROW,
            lg.FAMILY_GROUP_PER_ROW, lg.FAMILY_BATCHED, lg.FAMILY_BATCHED_MFMA]


def test_rounding_chain_bounded_for_long_rows():
    """bf16 1024 x 2^20 ran 2048 sequential multiply-adds into one
    accumulator; every plan now keeps at most 150 roundings between a
    product and its output (the tolerance's 1e-5 allows 167)."""
    q = lg.plan("bf16", 1024, 1 << 20, A_addr=ALIGNED, X_addr=ALIGNED)
    assert q["family"] == lg.FAMILY_GROUP_PER_ROW
    assert q["rounding_chain"] <= 150
    checked = 0
    for dtype in ("f32", "f16", "bf16"):
        for M in (1, 7, 64, 300, 1024, 4096, 1 << 16):
            for K in (1, 16, 100, 1000, 4096, 14336, 65536, 1 << 20, 1 << 24):
                if M * K > 1 << 36:
                    continue
                for fam in FAMILIES:
                    for nvec in ((1,) if fam < lg.FAMILY_BATCHED else (2, 16, 17, 33, 64)):
                        for A in (ALIGNED, ALIGNED + 4):
                            try:
                                q = lg.plan(dtype, M, K, K, nvec, A, A, fam)
                            except lg.GemvError:
                                continue
                            assert 1 <= q["rounding_chain"] <= 150, (dtype, M, K, fam, nvec, q)
                            checked += 1
    assert checked > 1000
    # split-K: pass 1 over a slice plus the reduce
    for dtype, M, K in (("f32", 8, 1 << 21), ("bf16", 64, 1 << 18), ("f16", 1, 1 << 24),
                        ("bf16", 1, (1 << 31) - 8)):
        q = lg.plan_splitk(dtype, M, K, A_addr=ALIGNED, x_addr=ALIGNED)
        assert q["rounding_chain"] <= 150, (dtype, M, K, q)


def _sum2_roundings(n):
    """Roundings a compensated running sum of n terms adds (one rounding plus
    gamma_{n-1}^2 / u, Ogita-Rump-Oishi Sum2), written out independently."""
    if n <= 1:
        return 0
    u = 2.0 ** -24
    g = (n - 1) * u / (1 - (n - 1) * u)
    return 1 + math.ceil(g * g / u - 1e-6)


def _batched_schedule_chain(K, E, B, RUN, KS):
    """Walk the vector-ALU batched kernel's schedule lane by lane: blocks of
    B*64 chunks dealt to KS wavefronts in turn, a wavefront's 64 lanes taking
    chunks c0 + 64*i + lane (i < B) of each of its blocks, products into one
    accumulator for RUN blocks before a compensated add, the element-wise
    tail (wavefront 0) as one more term; then the 64-lane tree and the fold
    of KS totals.  Returns the most roundings any product meets."""
    nfull = K // E
    tail = K - nfull * E
    worst = 0
    for w in range(KS):
        blocks = list(range(w * B * 64, nfull, KS * B * 64))
        terms = -(-len(blocks) // RUN) + (1 if tail and w == 0 else 0)
        for lane in (0, 63):
            longest = 0
            for r in range(0, len(blocks), RUN):
                run = sum(E for c0 in blocks[r:r + RUN] for i in range(B)
                          if c0 + 64 * i + lane < nfull)
                longest = max(longest, run)
            if w == 0 and tail:
                longest = max(longest, len(range(lane, tail, 64)))
            worst = max(worst, longest + _sum2_roundings(terms))
    return worst + 6 + (KS - 1)


def test_batched_chain_covers_the_kernel_schedule():
    """The vector-ALU batched plan's rounding chain is never below what its
    kernel's schedule makes a product meet (plus one for the bias), for
    every vector count's batch and run length, with and without the K
    split, on row lengths around the block and run boundaries."""
    checked = 0
    for dtype in ("f16", "bf16"):
        for M in (64, 1024, 4096):  # K over 4 or 2 wavefronts, and a wavefront per row
            for nvec in (2, 5, 9, 16):
                for K in (1, 7, 8, 100, 1023, 1024, 2047, 2048, 4096, 4100, 8191, 8200, 16384,
                          16391, 65536, 100003):
                    for A in (ALIGNED, ALIGNED + 2):
                        q = lg.plan(dtype, M, K, K, nvec, A, A, lg.FAMILY_BATCHED)
                        E = q["chunk_elems"]
                        B = q["batch"]
                        RUN = 1 if nvec <= 8 or B * E >= 64 else 64 // (B * E)
                        KS = q["lanes_per_row"] // 64
                        assert KS == (4 if M <= 512 else (2 if M <= 1536 and nvec >= 4 else 1))
                        need = _batched_schedule_chain(K, E, B, RUN, KS) + 1
                        assert q["rounding_chain"] >= need, (dtype, M, K, nvec, A, q, need)
                        assert q["rounding_chain"] <= 150
                        checked += 1
    assert checked == 2 * 3 * 4 * 16 * 2


def test_forced_wave_per_row_on_huge_rows():
    """A forced family whose chain would pass the bound is refused; the
    compensated running sum keeps even a wavefront per row of 2^24 elements
    within it."""
    q = lg.plan("bf16", 4, 1 << 24, family=lg.FAMILY_WAVE_PER_ROW, A_addr=ALIGNED, X_addr=ALIGNED)
    assert q["rounding_chain"] <= 150


def test_wide_batches_of_long_rows_run_in_blocks():
    """With 33-64 vectors the matrix-core kernel accumulates in place; rows
    long enough to push that chain past the bound run the vectors as blocks
    of 32 (two passes over A), each with compensated chunk sums."""
    short = lg.plan("bf16", 4096, 4096, nvec=64, A_addr=ALIGNED, X_addr=ALIGNED)
    assert short["column_blocks"] == 1 and short["rounding_chain"] <= 150
    long_ = lg.plan("bf16", 512, 1 << 17, nvec=64, A_addr=ALIGNED, X_addr=ALIGNED)
    assert long_["family"] == lg.FAMILY_BATCHED_MFMA
    assert long_["column_blocks"] == 2 and long_["rounding_chain"] <= 150
    assert lg.plan("bf16", 512, 1 << 17, nvec=40, A_addr=ALIGNED, X_addr=ALIGNED)["column_blocks"] == 2
    assert lg.plan("bf16", 512, 1 << 17, nvec=32, A_addr=ALIGNED, X_addr=ALIGNED)["column_blocks"] == 1
    assert lg.plan("bf16", 512, 1000, nvec=40, A_addr=ALIGNED + 2)["column_blocks"] == 3
