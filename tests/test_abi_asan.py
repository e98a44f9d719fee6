"""libaqua's host code under AddressSanitizer, without a GPU.

Every HIP source is compiled with the sanitizer on its host pass only (``-Xarch_host`` before
each sanitizer flag: the device code is not instrumented), linked with tests/abi_host_check.c
into one executable, and run: the size queries, and every entry point with arguments it must
reject before any HIP call, each rejection's error text read in full (the thread-local message
buffer is formatted by the library).  A heap or stack overflow, or a use after free, in that
host code aborts the run with the sanitizer's report."""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_dimension_attention_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, r.stdout + r.stderr


def test_abi_host_code_under_asan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    flags = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=1", *HOST_ASAN,
             f"-I{CSRC}", f"-I{INCLUDE}"]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]
    cmds = [[HIPCC, *flags, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    harness = str(tmp_path / "abi_host_check.o")
    cmds.append([HIPCC, "-x", "c", "-std=c99", "-O1", *HOST_ASAN, f"-I{INCLUDE}", "-c",
                 os.path.join(ROOT, "tests", "abi_host_check.c"), "-o", harness])
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        assert rc == 0, f"{' '.join(cmd)}\n{out[-2000:]}"
    exe = str(tmp_path / "abi_host_check")
    rc, out = _run([HIPCC, "--offload-arch=gfx950", *HOST_ASAN, *objs, harness, "-o", exe])
    assert rc == 0, out[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.strip().endswith("ok"), r.stdout
