"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  api.cpp is compiled with the sanitizers on its host pass (its
device code is built as usual) and linked with the library's other objects
and tests/sanitize/abi_driver.cpp, which drives every validation path, the
per-thread timing state from two threads and the no-allocation entry
point's size check; any sanitizer report fails the run.  The oracle is
numpy code (no native code of this project), so only the library's native
host code is instrumented here."""
import os
import shutil
import subprocess

import pytest

from transformer_ffn_block_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not installed")
def test_abi_host_code_is_sanitizer_clean():
    objs = [os.path.join(B.BUILD, s + ".o") for s in B.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    os.makedirs(OUT, exist_ok=True)
    inc = os.path.join(ROOT, "include")
    api_o, drv_o, exe = (os.path.join(OUT, n) for n in ("api.o", "driver.o", "abi_driver"))
    # the sanitizers instrument the host pass only (each flag behind -Xarch_host)
    _run([B.hipcc(), "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
          "-I", inc, "-c", os.path.join(B.CSRC, "api.cpp"), "-o", api_o])
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    _run([CLANG, "-O1", "-g", "-std=c++17", *san, "-I", inc, "-c",
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv_o])
    _run([CLANG, *san, drv_o, api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
          "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "abi driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    shutil.rmtree(OUT, ignore_errors=True)
