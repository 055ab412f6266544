"""libgemv calls captured in a HIP graph (needs a GPU).

The library allocates nothing, sets no memory and only enqueues kernels on
the caller's stream, so its calls can be recorded in a graph and replayed.
Each replay is checked against the same calls run eagerly, bit for bit,
with the program's own eager work and synchronisations between replays."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gemv_inputs as gi
import memory_bound_gemv_f32_amd as lg
from gpu_helpers import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs():
    """Device inputs for one call of every entry point family."""
    dev = {}
    c = gi.make_random("bf16", 4096, 4096, seed=1, dist="normal", scale=0.02, bias=True)
    dev["A"] = to_device("bf16", c.A.reshape(c.M, c.lda))
    dev["x"] = to_device("bf16", c.X[0])
    dev["bias"] = torch.from_numpy(c.bias).cuda()
    b = gi.make_random("f16", 1000, 2048, seed=2, nvec=24, dist="normal")
    dev["Ab"] = to_device("f16", b.A.reshape(b.M, b.lda))
    dev["Xb"] = to_device("f16", b.X)
    b2 = gi.make_random("bf16", 1000, 2050, seed=7, nvec=5, dist="normal")  # K % 8 != 0
    dev["Ab2"] = to_device("bf16", b2.A.reshape(b2.M, b2.lda))
    dev["Xb2"] = to_device("bf16", b2.X)
    s = gi.make_random("f32", 8, 1 << 18, seed=3)
    dev["As"] = to_device("f32", s.A.reshape(s.M, s.lda))
    dev["xs"] = to_device("f32", s.X[0])
    n = lg.splitk_workspace_size("f32", s.M, s.K)
    dev["ws"] = torch.empty(max(n // 4, 1), dtype=torch.float32, device="cuda")
    q, k, v = (gi.make_random("bf16", M, 4096, seed=10 + M, dist="normal", scale=0.02)
               for M in (512, 128, 128))
    dev["qkv"] = [to_device("bf16", t.A.reshape(t.M, t.lda)) for t in (q, k, v)]
    g = gi.make_random("bf16", 1024, 4096, seed=4, dist="normal", scale=0.02)
    u = gi.make_random("bf16", 1024, 4096, seed=5, dist="normal", scale=0.02)
    dev["Ag"] = to_device("bf16", g.A.reshape(g.M, g.lda))
    dev["Au"] = to_device("bf16", u.A.reshape(u.M, u.lda))
    b3 = gi.make_random("bf16", 300, 2050, seed=8, nvec=12, dist="normal")  # K split over 4 wavefronts
    dev["Ab3"] = to_device("bf16", b3.A.reshape(b3.M, b3.lda))
    dev["Xb3"] = to_device("bf16", b3.X)
    b4 = gi.make_random("f16", 13313, 1024, seed=9, nvec=12, dist="normal")  # 32-row MFMA workgroups
    dev["Ab4"] = to_device("f16", b4.A.reshape(b4.M, b4.lda))
    dev["Xb4"] = to_device("f16", b4.X)
    w = gi.make_q8_random("f16", 2048, 4096, seed=6)
    dev["Q"] = torch.from_numpy(w.Q).cuda()
    dev["scale"] = torch.from_numpy(w.scale).cuda()
    dev["xq"] = to_device("f16", w.X[0])
    return dev


def _outputs():
    return {
        "y": torch.empty(4096, device="cuda"),
        "Y": torch.empty((24, 1000), device="cuda"),
        "Y2": torch.empty((5, 1000), device="cuda"),
        "Y3": torch.empty((12, 300), device="cuda"),
        "Y4": torch.empty((12, 13313), device="cuda"),
        "yn": torch.empty(8, device="cuda"),
        "ys": torch.empty(8, device="cuda"),
        "yqkv": [torch.empty(M, device="cuda") for M in (512, 128, 128)],
        "h": torch.empty(1024, device="cuda"),
        "yq": torch.empty(2048, device="cuda"),
    }


def _calls(d, o):
    """One call of each entry point family, on the current stream."""
    lg.gemv(d["A"], d["x"], d["bias"], out=o["y"])
    lg.gemv_batched(d["Ab"], d["Xb"], out=o["Y"])
    lg.gemv_splitk(d["As"], d["xs"], out=o["ys"], workspace=d["ws"])
    lg.gemv_batched(d["Ab2"], d["Xb2"], out=o["Y2"])  # the vector-ALU batched kernel
    lg.gemv_batched(d["Ab3"], d["Xb3"], out=o["Y3"])  # ... with each row's K split
    lg.gemv_batched(d["Ab4"], d["Xb4"], out=o["Y4"])  # matrix cores, four row groups
    rc = lg.gemv_splitk_noalloc(lg.DTYPE_F32, d["As"].data_ptr(), d["As"].stride(0),
                                d["xs"].data_ptr(), None, o["yn"].data_ptr(), d["As"].shape[0],
                                d["As"].shape[1], 0, torch.cuda.current_stream().cuda_stream)
    assert rc == lg.GEMV_SUCCESS
    lg.gemv_multi(d["qkv"], d["x"], None, o["yqkv"])
    lg.gemv_gate_up_silu(d["Ag"], d["Au"], d["x"], out=o["h"])
    lg.gemv_q8(d["Q"], d["scale"], d["xq"], out=o["yq"])


def _flat(o):
    parts = [o["y"], o["Y"].reshape(-1), o["ys"], o["Y2"].reshape(-1), o["Y3"].reshape(-1),
             o["Y4"].reshape(-1), o["yn"], *o["yqkv"], o["h"], o["yq"]]
    return torch.cat([p.reshape(-1) for p in parts]).cpu().numpy()


def test_captured_calls_replay_like_eager_ones():
    d = _inputs()
    eager = _outputs()
    _calls(d, eager)
    torch.cuda.synchronize()
    want = _flat(eager)
    assert np.isfinite(want).all()
    # the forms these calls are meant to reach
    assert lg.plan("bf16", 300, 2050, 2050, 12, d["Ab3"].data_ptr(), d["Xb3"].data_ptr())["lanes_per_row"] == 256
    assert lg.plan("f16", 13313, 1024, 1024, 12, d["Ab4"].data_ptr(), d["Xb4"].data_ptr())["row_tiles"] == 4
    # the allocation-free split-K gives the workspace split-K's bits
    assert torch.equal(eager["yn"], eager["ys"])

    out = _outputs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _calls(d, out)  # warm the launch path outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _calls(d, out)
    torch.cuda.synchronize()
    for replay in range(3):
        for t in (out["y"], out["Y"], out["ys"], out["Y2"], out["Y3"], out["Y4"], out["yn"],
                  *out["yqkv"], out["h"], out["yq"]):
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _flat(out)
        assert np.array_equal(got, want), f"replay {replay} differs from the eager calls"
