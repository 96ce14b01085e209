"""The library's host code under the address and undefined-behaviour
sanitizers, on the CPU: every source is compiled host-only (the device code
is not built), linked with a host-only stand-in for the HIP runtime
(tests/sanitize/fake_hip.cpp) that records kernel launches instead of
running them, and driven through every C ABI entry point by
tests/sanitize/abi_driver.cpp: rejected arguments launch nothing, accepted
ones launch kernels within a gfx950 launch's limits, the size queries
survive fuzzing with sizes of every magnitude, and the host fp64 routines
give the values their definitions fix."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from compressed_gemv_amd import build as qbuild

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = os.path.join(HERE, "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"

pytestmark = pytest.mark.skipif(not (os.path.exists(CLANG) and shutil.which("nm")), reason="clang++ or nm missing")

# sanitizer flags for the host side of a HIP compile: each one after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_host_code_sanitized(tmp_path):
    cc = qbuild.hipcc()
    objs = []

    def compile_one(src):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        _run([cc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-host-only", f"--offload-arch={qbuild.ARCH}",
              *HOST_SAN, "-Wno-unused-command-line-argument", "-I", qbuild.INCLUDE, "-I", qbuild.CSRC,
              "-c", os.path.join(qbuild.CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, qbuild.SOURCES))
    # a host-only object refers to its (absent) device image by name; give each one an empty image
    names = set()
    for o in objs:
        for line in _run(["nm", "-u", o]).stdout.splitlines():
            sym = line.split()[-1]
            if sym.startswith("__hip_fatbin_"):
                names.add(sym)
    stub = tmp_path / "images.cpp"
    stub.write_text("".join(f'extern "C" const char {n}[64] = {{0}};\n' for n in sorted(names)))
    exe = str(tmp_path / "abi_driver")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", qbuild.INCLUDE,
          "-I", SAN, os.path.join(SAN, "fake_hip.cpp"), os.path.join(SAN, "abi_driver.cpp"), str(stub), *objs, "-o", exe, "-lm", "-lpthread"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-8000:]
    assert " 0 failed" in r.stdout and "Sanitizer" not in r.stderr, r.stderr[-8000:]
