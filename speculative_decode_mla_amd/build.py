"""Build libmla_verify.so for gfx950 with hipcc (in-tree, next to this file).

    python -m speculative_decode_mla_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmla_verify.so")
# the same sources with the device-side argument checks compiled in (MLA_VERIFY_DEBUG)
DEBUG_LIB = os.path.join(HERE, "libmla_verify_debug.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("mla_verify_api.hip", "mla_verify_kernels.hip", "mla_kv_compact.hip", "mla_step_metadata.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17",
    # keep packed fp32 VALU ops out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the leading kernel arguments (kernel 1's lengths and sizes) arrive in scalar registers
    "-mllvm", "-amdgpu-kernarg-preload-count=7",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]


def device_asm(source: str, out_path: str) -> str:
    """gfx950 assembly of one source file with the library's flags (for inspection and checks)."""
    cmd = [hipcc(), *COMMON_FLAGS, "--cuda-device-only", "-S", source, "-o", out_path]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed ({r.returncode}):\n{r.stderr}")
    return out_path


def build(verbose: bool = False) -> str:
    """Compile the release and the debug library; returns the release library's path.  Always recompiles."""
    _build_one(LIB, [], verbose)
    _build_one(DEBUG_LIB, ["-DMLA_VERIFY_DEBUG"], verbose)
    return LIB


def _build_one(path: str, defines, verbose: bool) -> str:
    tmp = path + ".tmp"
    cmd = [hipcc(), *COMMON_FLAGS, *defines, "-fPIC", "-shared", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, path)
    return path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
