"""The built library's gfx950 code object, read from its own metadata (no
GPU): every kernel runs without scratch memory (no spilled registers, no
private arrays, no dynamic stack) and within the LDS and register limits
the launches assume.  A kernel that starts to spill after a change fails
here instead of silently running several times slower."""

from __future__ import annotations

import re
import shutil
import subprocess
from pathlib import Path

import pytest

import memory_bound_gemv_f32_amd as lg

LLVM = Path("/opt/rocm/llvm/bin")
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
LDS_BYTES = 160 * 1024


def _tool(name: str) -> str:
    path = LLVM / name
    if path.exists():
        return str(path)
    found = shutil.which(name)
    if found is None:
        pytest.skip(f"{name} not available")
    return found


@pytest.fixture(scope="module")
def kernels(tmp_path_factory) -> list[dict]:
    """Per-kernel metadata of the gfx950 code object inside libgemv.so."""
    tmp = tmp_path_factory.mktemp("code_object")
    fatbin, obj = tmp / "fatbin.bin", tmp / "gfx950.o"
    subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fatbin}",
                    str(lg.LIBRARY), str(tmp / "host.discard")], check=True, capture_output=True)
    subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--targets={TARGET}",
                    f"--input={fatbin}", f"--output={obj}"], check=True, capture_output=True)
    notes = subprocess.run([_tool("llvm-readelf"), "--notes", str(obj)], check=True,
                           capture_output=True, text=True).stdout
    out, cur = [], None
    # each kernel's entry starts at its argument list ("- .agpr_count" or
    # "- .args"); the scalar fields follow at the entry's own indentation
    for line in notes.splitlines():
        m = re.match(r"\s*(?:- )?\.(\w+):\s*(\S+)?\s*$", line)
        if not m:
            continue
        key, value = m.group(1), m.group(2)
        if line.lstrip().startswith("- .") and key in ("agpr_count", "args") and line.startswith("  - "):
            cur = {}
            out.append(cur)
        if cur is not None and value is not None and key in (
                "name", "private_segment_fixed_size", "group_segment_fixed_size", "vgpr_count",
                "agpr_count", "sgpr_spill_count", "vgpr_spill_count", "uses_dynamic_stack",
                "max_flat_workgroup_size", "wavefront_size"):
            cur.setdefault(key, value)
    return [k for k in out if "name" in k]


def test_every_kernel_is_listed(kernels):
    names = [k["name"] for k in kernels]
    assert len(names) > 1000 and len(set(names)) == len(names)
    for family in ("gemv_rows_kernel", "gemv_group_kernel", "gemv_group_stream_kernel",
                   "gemv_batched_kernel", "gemv_batched_mfma_kernel", "gemv_gated_silu_kernel",
                   "gemv_splitk_partial_kernel", "gemv_splitk_reduce_kernel", "gemv_rows_q8_kernel",
                   "gemv_group_q8_kernel", "gemv_group_stream_q8_kernel"):
        assert any(family in n for n in names), family


def test_no_kernel_uses_scratch(kernels):
    bad = [k["name"] for k in kernels
           if k.get("private_segment_fixed_size") != "0" or k.get("vgpr_spill_count") != "0"
           or k.get("sgpr_spill_count") != "0" or k.get("uses_dynamic_stack") != "false"]
    assert not bad, f"{len(bad)} kernels use scratch memory, e.g. {bad[:3]}"


def test_resources_fit_the_launches(kernels):
    for k in kernels:
        assert k["wavefront_size"] == "64", k["name"]
        assert int(k["group_segment_fixed_size"]) <= LDS_BYTES, k["name"]
        waves = int(k["max_flat_workgroup_size"]) // 64
        # a workgroup's wavefronts share the SIMDs' 512 registers per lane
        simd_waves = max(1, -(-waves // 4))
        assert int(k["vgpr_count"]) + int(k.get("agpr_count", "0")) <= 512 // simd_waves, k["name"]
