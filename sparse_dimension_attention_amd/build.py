"""Builds libaqua.so in-tree with hipcc for gfx950 (the only target).

Every HIP source is compiled to an object of its own, in parallel (the decode kernel templates
are instantiated in several translation units so that no one of them dominates), then the
objects are linked into the shared library.  Objects go to ``_build/`` next to the package.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OUT = os.path.join(HERE, "libaqua.so")
OBJ_DIR = os.path.join(os.path.dirname(HERE), "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the attention's O is rescaled by VALU between MFMAs
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]
LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC"]
NOISE = "is not a recognized feature for this target"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if NOISE not in l)
    return res.returncode, msgs


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source and link libaqua.so; returns its path.  Always recompiles."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s) + ".o") for s in srcs]
    cmds = [[HIPCC, *COMPILE_FLAGS, f"-I{CSRC}", f"-I{INCLUDE}", "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    errors = [(c, m) for c, (rc, m) in zip(cmds, results) if rc != 0]
    if errors:
        raise RuntimeError("\n\n".join(f"hipcc failed:\n{' '.join(c)}\n{m}" for c, m in errors))
    if verbose:
        for (_, m) in results:
            if m.strip():
                print(m)
    tmp = OUT + ".tmp"
    rc, msgs = _run([HIPCC, *LINK_FLAGS, *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{msgs}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
