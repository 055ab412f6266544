"""A seeded sweep through the automatic planner on the GPU: single-vector,
batched and int8-weight calls whose row counts sit on the planner's
boundaries (one workgroup per compute unit and just past it, the 2- and
4-wavefront workgroup choices, the matrix-core row groups, the int8
workgroup shapes), on exact-integer data: every result bit-exact against
the oracle."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gemv_inputs as gi
import memory_bound_gemv_f32_amd as lg
from gpu_helpers import assert_bit_exact, run_gpu, run_oracle
from test_q8_gpu import run_oracle_q8, run_q8

pytestmark = pytest.mark.gpu

ROWS = [1, 3, 9, 33, 255, 257, 511, 513, 1021, 1024, 1025, 1280, 1535, 1536, 2047, 2048, 2049,
        2304, 2560, 3584, 4095, 4096, 4097, 4113, 6144, 8192, 14336, 16383, 16384, 16385, 65537]
ROW_BYTES = [16, 48, 256, 520, 1024, 2048, 4096, 5000, 8192, 8208, 12288, 16400, 28672]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_seeded_sweep_every_path():
    rng = np.random.default_rng(1234)
    done, kinds = 0, {}
    while done < 400:
        kind = str(rng.choice(["single", "single", "batched", "int8"]))
        M = int(rng.choice(ROWS))
        if kind == "int8":
            xd = str(rng.choice(gi.DTYPES))
            K = int(rng.choice([16, 100, 256, 1000, 4096, 4100, 8192, 11008]))
            if M * K > 80_000_000:
                continue
            ldq = K + int(rng.choice([0, 0, 3, 16]))
            case = gi.make_q8_integer(xd, M, K, seed=5000 + done, ldq=ldq,
                                      bias=bool(rng.integers(2)))
            q = lg.plan_q8(xd, M, K, ldq, 1 << 20, 1 << 20)
            what = (f"case {done}: int8 x {xd} {M}x{K} ldq={ldq}: {lg.FAMILY_NAMES[q['family']]}, "
                    f"{q['waves_per_group']} wavefronts, {q['row_tiles']} tiles")
            print(what, flush=True)
            ref, _ = run_oracle_q8(case)
            assert_bit_exact(run_q8(case), ref, what)
        else:
            dtype = str(rng.choice(gi.DTYPES if kind == "single" else ["f16", "bf16"]))
            es = gi.ELEMENT_BYTES[dtype]
            K = int(rng.choice(ROW_BYTES)) // es + int(rng.choice([0, 0, 0, 1, -1]))
            nvec = 1 if kind == "single" else int(rng.choice([2, 3, 5, 6, 8, 16, 17, 24, 33, 64]))
            if K < 1 or M * K * nvec > 150_000_000 or M * K > 80_000_000:
                continue
            lda = K + int(rng.choice([0, 0, 0, 1, 16 // es]))
            misalign = int(rng.choice([0, 0, 0, 1]))
            case = gi.make_integer(dtype, M, K, seed=9000 + done, nvec=nvec, lda=lda,
                                   bias=bool(rng.integers(2)))
            A_addr = (1 << 20) + (es if misalign else 0)
            q = lg.plan(dtype, M, K, lda, nvec, A_addr, A_addr)
            what = (f"case {done}: {dtype} {M}x{K} lda={lda} nvec={nvec} misalign={misalign}: "
                    f"{lg.FAMILY_NAMES[q['family']]}, {q['waves_per_group']} wavefronts, "
                    f"{q['rows_per_group']} rows per workgroup")
            print(what, flush=True)
            ref, _ = run_oracle(case)
            assert_bit_exact(run_gpu(case, lg.FAMILY_AUTO, misalign=misalign, batched=nvec > 1),
                             ref, what)
        kinds[kind] = kinds.get(kind, 0) + 1
        done += 1
    assert min(kinds.values()) >= 50, kinds
