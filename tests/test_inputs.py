"""The seeded input generators and the algorithmic byte model (no GPU)."""

import json
from pathlib import Path

import numpy as np
import torch

import gemv_inputs as gi

GOLDEN = Path(__file__).resolve().parent / "golden"


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    f = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, 3.4e38,
                                  1.0 + 2**-8, 1.0 + 3 * 2**-8], np.float32)])
    ours = gi.f32_to_bf16_bits(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ours, ref.view(np.uint16))
    nan = gi.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_f16_rounding_matches_torch():
    # binary32 inputs, so torch's cast (which goes through binary32) rounds once
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(100000) * 100).astype(np.float32)
    ours = gi.to_f16_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float16).view(torch.int16).numpy()
    assert np.array_equal(ours, ref.view(np.uint16))
    # float64 input just below a binary16 tie rounds down (no double rounding)
    assert gi.to_f16_bits(np.array([24.0234371511884]))[0] == 0x4E01


def test_generators_are_seeded_and_laid_out():
    a = gi.make_random("bf16", 33, 70, seed=5, nvec=3, lda=80, bias=True)
    b = gi.make_random("bf16", 33, 70, seed=5, nvec=3, lda=80, bias=True)
    assert np.array_equal(a.A, b.A) and np.array_equal(a.X, b.X)
    assert a.A.shape == (33, 80) and a.X.shape == (3, 70)
    assert a.A.dtype == np.uint16 and a.bias.dtype == np.float32
    assert np.all(a.A[:, 70:] == 0x7FC0)          # NaN padding
    c = gi.make_random("f32", 4, 5, seed=6, lda=8)
    assert np.all(np.isnan(c.A[:, 5:])) and not np.isnan(c.A[:, :5]).any()


def test_workload_table():
    assert gi.workload_shape("skinny_k16") == ("f32", 1 << 20, 16, 1, True)
    assert gi.workload_shape("batched_f16_4096x16") == ("f16", 4096, 4096, 16, False)
    assert gi.workload_shape("sweep_down") == ("bf16", 4096, 14336, 1, False)
    c = gi.make_workload("sgemv_1024x128")
    assert c.A.shape == (1024, 128) and c.bias is None
    assert c.A.min() >= -1 and c.A.max() <= 1


def test_byte_model_matches_pages():
    fx = json.loads((GOLDEN / "pages_byte_model.json").read_text())["entries"]
    # fp32: bytes 4MN + 4N + 4M and 2MN flops, intensity near 0.5
    for M, N in ((3, 1024), (4096, 4096), (1024, 128)):
        t = fx[0]["bytes_terms"]
        want = (t["A_per_element"] * M * N + t["x_per_element"] * N
                + t["y_per_element"] * M)
        assert gi.workload_bytes("f32", M, N) == want
        assert gi.workload_flops(M, N) == fx[0]["flops_per_MN"] * M * N
    ai = gi.workload_flops(4096, 4096) / gi.workload_bytes("f32", 4096, 4096)
    assert abs(ai - fx[0]["intensity_approx"]) < 1e-3
    # fp16 4096x4096, one vector: 33.6 MFLOP over about 33.6 MB, intensity ~1
    e = fx[2]
    flops = gi.workload_flops(e["M"], e["K"], e["vectors"])
    nbytes = gi.workload_bytes(e["dtype"], e["M"], e["K"], e["vectors"])
    assert round(flops / 1e6, 1) == e["flops_printed_M"]
    assert round(e["M"] * e["K"] * 2 / 1e6, 1) == e["weight_bytes_printed_MB"]
    assert abs(flops / nbytes - e["intensity_approx"]) < 1e-2
    # x@W with m rows and fp32 output instead of s-byte output
    m, k, n, s = 16, 4096, 4096, 2
    assert gi.workload_bytes("f16", n, k, m) == (m * k + k * n) * s + 4 * m * n


def test_q8_generators():
    c = gi.make_q8_random("bf16", 10, 100, seed=1, ldq=104, bias=True, nvec=2)
    assert c.Q.dtype == np.int8 and c.Q.shape == (10, 104)
    assert np.all(c.Q[:, 100:] == -128) and np.abs(c.Q[:, :100].astype(int)).max() <= 127
    assert c.scale.dtype == np.float32 and np.all(c.scale > 0)
    assert c.X.shape == (2, 100) and c.X.dtype == np.uint16
    assert c.algorithmic_bytes() == 10 * 100 + 4 * 10 + 2 * 100 * 2 + 4 * 10 * 2 + 4 * 10
    i = gi.make_q8_integer("f16", 300, 50, seed=2)
    assert set(np.unique(i.Q)) <= set(range(-128, 128)) and i.Q.min() == -128 and i.Q.max() == 127
    assert np.all(np.log2(i.scale) == np.round(np.log2(i.scale)))
    w = gi.make_q8_workload("q8_f16_4096")
    assert (w.M, w.K, w.xdtype) == (4096, 4096, "f16")
    assert w.algorithmic_bytes() == 4096 * 4096 + 4 * 4096 + 2 * 4096 + 4 * 4096
