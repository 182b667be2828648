"""Build the HIP library (libsplash_attn.so) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import tempfile
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libsplash_attn.so"
SOURCES = ["abi.hip", "kv_append.hip", "verify_attn.hip", "accept.hip"]
# measurement probe used by bench.py only (not part of the attention library)
PROBE_LIB = PKG / "libsplash_probe.so"
PROBE_SOURCES = ["read_ceiling.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # never form packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: no AGPR is used, which gives a wave the whole register budget as VGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]

# Per-source flags.  The attention kernels never rely on NaN semantics of
# min/max (masked scores are -inf, chosen by integer compares; infinities stay
# honoured), so their max needs no operand canonicalisation.  The quantiser
# keeps strict IEEE fp32.
SOURCE_FLAGS = {
    "verify_attn.hip": ["-fno-honor-nans"],
}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = Path(rocm) / "bin" / "hipcc"
    return str(cand) if cand.exists() else "hipcc"


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + proc.stderr[-6000:])


def build(out: Path = LIB, extra_flags=(), sources=None) -> Path:
    """Compile every HIP source and link one shared library (always recompiles)."""
    tmp = Path(str(out) + ".tmp")
    with tempfile.TemporaryDirectory(prefix="splash_build_") as td:
        objs = []
        for src in (SOURCES if sources is None else sources):
            obj = Path(td) / (Path(src).stem + ".o")
            _run([hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, "-c", str(CSRC / src),
                  "-o", str(obj)])
            objs.append(str(obj))
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp), *objs])
    os.replace(tmp, out)
    return out


def build_probe() -> Path:
    """The bandwidth probe library bench.py reports the practical read ceiling with."""
    return build(PROBE_LIB, sources=PROBE_SOURCES)


if __name__ == "__main__":
    print(build())
    print(build_probe())
