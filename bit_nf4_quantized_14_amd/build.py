"""Build the HIP library ``libqlora_nf4.so`` in-tree for gfx950.

``python -m bit_nf4_quantized_14_amd.build`` (or ``__graft_entry__.build()``)
compiles every source under ``csrc/`` with hipcc and writes the shared
library next to this file, where :mod:`bit_nf4_quantized_14_amd.capi` loads
it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libqlora_nf4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def compile_command(out: str = LIB_PATH) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-shared", "-Wall", "-Wno-unused-function",
        # keep packed-fp32 instructions out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *sources(), "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always; no up-to-date check) and return its
    path."""
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
