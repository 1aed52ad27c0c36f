"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C-ABI library is rebuilt with its host code instrumented (hipcc,
-Xarch_host before each sanitizer flag, so the gfx950 code is the product's
own), the float64 oracle is rebuilt with clang under the same sanitizers, and
the CPU suite runs against both in a child process with the sanitizer
runtime preloaded.  This is the host-side counterpart of the memcheck and
racecheck runs over the slice cases (TensorFold pull request #1355,
follow-up checks).  Any sanitizer report fails the test; so does a child
that did not load both instrumented libraries."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"

CHILD = r"""
import sys
import pytest
import paged_kv_cache_addressing_amd as pa
import oracle
pa.LIB_PATH = sys.argv[1]
oracle.LIB = sys.argv[2]
rc = pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                  "--deselect", "tests/test_host_sanitizers.py", "tests"])
maps = open("/proc/self/maps").read()
print("LOADED", sys.argv[1] in maps, sys.argv[2] in maps)
sys.exit(rc)
"""


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and _asan_runtime()),
                    reason="hipcc, clang or the clang ASan runtime is missing")
def test_cpu_suite_is_clean_under_asan_and_ubsan(tmp_path):
    from paged_kv_cache_addressing_amd import build as B
    csrc = os.path.join(ROOT, "paged_kv_cache_addressing_amd", "csrc")
    # host-only instrumentation: every sanitizer flag behind its own -Xarch_host
    san_link = ["-Xarch_host", "-fsanitize=address",
                "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-shared-libasan"]
    san = san_link + ["-Xarch_host", "-fno-sanitize-recover=undefined",
                      "-fno-omit-frame-pointer", "-g"]
    flags = [f for f in B.COMMON if f != "-O3"] + ["-O1"]
    lib = str(tmp_path / "libpaged_attn_san.so")
    objs = [str(tmp_path / (src + ".o")) for src in B.SOURCES]

    def compile_one(i):
        src = B.SOURCES[i]
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        subprocess.run([HIPCC] + flags + san + lang + B.EXTRA.get(src, []) +
                       ["-c", os.path.join(csrc, src), "-o", objs[i]], check=True,
                       stderr=subprocess.DEVNULL)
    with ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(compile_one, range(len(B.SOURCES))))
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + san_link +
                   ["-o", lib] + objs, check=True, stderr=subprocess.DEVNULL)
    olib = str(tmp_path / "liboracle_san.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-D_POSIX_C_SOURCE=200809L", "-fPIC",
                    "-shared", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-shared-libasan", "-o", olib,
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-lpthread"], check=True)
    env = dict(os.environ)
    env.update(PYTHONPATH=ROOT, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", CHILD, lib, olib], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "LOADED True True" in out, out[-2000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
