"""Build the HIP library in-tree for gfx950.

``python -m bit_nf4_quantized_14_amd.build`` (or ``__graft_entry__.build()``)
compiles every source under ``csrc/`` with hipcc (one object per source, in
parallel) and links two shared libraries next to this file:

* ``libqlora_nf4.so``      -- the library (:mod:`bit_nf4_quantized_14_amd.capi`
  loads it by default);
* ``libqlora_nf4_prof.so`` -- the same sources built with QN_PROFILE_HOOK,
  whose ``qn_profile_kernel`` records HIP events around one named kernel's
  launches (used by bench.py).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libqlora_nf4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
PROF_LIB_PATH = os.path.join(PKG_DIR, "libqlora_nf4_prof.so")
ARCH = "gfx950"
VARIANTS = {LIB_PATH: [], PROF_LIB_PATH: ["-DQN_PROFILE_HOOK"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def compile_flags(defines: list[str]) -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        # keep packed-fp32 instructions out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", f"-I{CSRC}", *defines,
    ]


def compile_command(src: str, obj: str, defines: list[str]) -> list[str]:
    return [hipcc(), *compile_flags(defines), "-c", src, "-o", obj]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" +
                           res.stdout + res.stderr)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile both library variants (always; no up-to-date check) and
    return the path of the default one."""
    jobs = jobs or max(1, min(8, os.cpu_count() or 1))
    srcs = sources()
    plan = []        # (lib, objects, compile commands)
    for lib, defines in VARIANTS.items():
        tag = os.path.splitext(os.path.basename(lib))[0]
        odir = os.path.join(OBJ_DIR, tag)
        os.makedirs(odir, exist_ok=True)
        objs = [os.path.join(odir, os.path.basename(s) + ".o") for s in srcs]
        plan.append((lib, objs, [compile_command(s, o, defines)
                                 for s, o in zip(srcs, objs)]))
    cmds = [c for _, _, cs in plan for c in cs]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    for lib, objs, _ in plan:
        tmp = lib + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
              "-o", tmp], verbose)
        os.replace(tmp, lib)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
