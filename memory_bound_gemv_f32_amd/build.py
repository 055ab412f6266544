"""Build libgemv.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python memory_bound_gemv_f32_amd/build.py`` (a standalone script: it
does not import the package, whose import needs the built library);
``__graft_entry__.build`` loads this file by path and calls :func:`build`.
The library is written next to this file, in-tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PACKAGE = Path(__file__).resolve().parent
ROOT = PACKAGE.parent
CSRC = PACKAGE / "csrc"
SOURCES = [CSRC / "gemv_api.hip"]
HEADERS = [CSRC / "gemv_plan.hpp", CSRC / "gemv_device.hpp",
           CSRC / "gemv_kernels.hpp", ROOT / "include" / "gemv.h"]
LIBRARY = PACKAGE / "libgemv.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments arrive preloaded in SGPRs (gfx950), so a kernel's
    # first loads do not wait on scalar loads of its argument block
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = shutil.which("hipcc") or os.path.join(rocm, "bin", "hipcc")
    return path


def build(verbose: bool = False, extra_flags: list[str] | None = None,
          output: Path = LIBRARY) -> Path:
    """Compile every HIP source into ``libgemv.so`` (always recompiles)."""
    tmp = output.with_name(f"{output.name}.tmp{os.getpid()}")
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []),
           *[str(s) for s in SOURCES], "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning
    # is expected, anything else is shown
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines()
            if noise not in ln and "(ignoring feature)" not in ln and ln.strip()]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, output)
    return output


def is_stale() -> bool:
    if not LIBRARY.exists():
        return True
    t = LIBRARY.stat().st_mtime
    return any(p.stat().st_mtime > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    build(verbose=True)
    print(LIBRARY)
