"""Build the HIP library (libsplash_attn.so) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libsplash_attn.so"
SOURCES = ["abi.hip", "kv_append.hip", "verify_attn.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # never form packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs, which leaves the AGPRs to the query operands
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = Path(rocm) / "bin" / "hipcc"
    return str(cand) if cand.exists() else "hipcc"


def build(out: Path = LIB, extra_flags=()) -> Path:
    """Compile every HIP source into one shared library (always recompiles)."""
    tmp = Path(str(out) + ".tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-o", str(tmp), *[str(CSRC / s) for s in SOURCES]]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stderr[-6000:])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
