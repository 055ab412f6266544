"""bench.py's host-side logic (no GPU): CLI contract, counter summary, and
the source hash that guards stored counter figures."""

import csv
import json
import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parent.parent


def _write_counters(d: Path, counter: str, gemv_vals, copy_vals):
    d.mkdir(parents=True, exist_ok=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for v in copy_vals:
            w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter, "Counter_Value": v})
        for v in gemv_vals:
            w.writerow({"Kernel_Name": "void gemvdev::gemv_rows_kernel<...>", "Counter_Name": counter,
                        "Counter_Value": v})


def test_summarize_counters_scales_by_the_copy(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    _write_counters(tmp_path / "f", "FETCH_SIZE", [100.0, 102.0], [5.0, copy_kib / 2])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [8.0, 8.0], [1.0, copy_kib])
    t = bench.summarize_counters(tmp_path / "f", tmp_path / "w", "sweep_q")
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["fetch_bytes_per_launch"] == 101.0 * 1024 * 2
    assert t["traffic_bytes_per_launch"] == 101.0 * 2048 + 8 * 1024
    assert t["source_hash"] == bench.kernel_source_hash()


def test_source_hash_is_stable_and_guards_traffic(tmp_path, monkeypatch):
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = bench.traffic_file("w")
    json.dump({"source_hash": "not-this-one", "traffic_bytes_per_launch": 1}, open(path, "w"))
    assert bench.load_traffic("w") is None
    json.dump({"source_hash": bench.kernel_source_hash(), "traffic_bytes_per_launch": 1}, open(path, "w"))
    assert bench.load_traffic("w")["traffic_bytes_per_launch"] == 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_fused_bytes_of_the_named_and_sharded_layers():
    import gemv_inputs as gi
    assert bench.fused_bytes("fused_qkv", gi.make_fused_qkv(), gi) == gi.fused_qkv_bytes()
    assert bench.fused_bytes("fused_gate_up", list(gi.make_fused_gate_up()), gi) == \
        gi.fused_gate_up_bytes()
    # a row shard: 1/8 of the rows, the same x
    parts = [gi.make_random("bf16", M // 8, K, seed=1) for M, K in ((4096, 4096), (1024, 4096))]
    assert bench.fused_bytes("fused_qkv", parts, gi) == (512 + 128) * 4096 * 2 + 4096 * 2 + 4 * 640


def test_source_hash_ignores_comments_and_layout():
    code = 'int f(int a) {\n  return a + 1;  // one more\n}\n/* note */ const char* s = "// not a comment";\n'
    same = 'int f(int a) { return a + 1;\n}   const char* s = "// not a comment";'
    assert bench.source_code_only(code) == bench.source_code_only(same)
    assert bench.source_code_only("a = 1; // x") != bench.source_code_only("a = 2; // x")
    assert '"// not a comment"' in bench.source_code_only(code)
    assert bench.source_code_only("x /* a */ y") == "x y"
