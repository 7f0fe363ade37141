"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

``mla_api.cpp`` (argument validation, the slot-coverage check, the error
buffer) is compiled by g++ with ``-fsanitize=address,undefined`` and linked
with the library's HIP objects (their host side: launch stubs and code-object
registration, not instrumented) into a separate shared library.  The ABI tests
then run against it in a child process with the sanitizer runtimes preloaded;
any report fails the child.  CPU only: no kernel is launched.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mla_latent_cache_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("gcc sanitizer runtimes or the HIP headers are not installed")
    from mla_latent_cache_amd import build as B
    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    d = tmp_path_factory.mktemp("asan")
    obj = str(d / "mla_api_asan.o")
    lib = str(d / "libmla_latent_asan.so")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", *san,
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(PKG, "csrc", "mla_api.cpp"), "-o", obj], check=True)
    subprocess.run(["g++", "-shared", *san, "-o", lib, obj, *objs, "-L", os.path.join(ROCM, "lib"),
                    "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64"], check=True)
    return lib, asan, ubsan


def test_abi_tests_under_asan_ubsan(asan_lib):
    lib, asan, ubsan = asan_lib
    env = dict(os.environ)
    env.update(MLA_LATENT_LIB=lib, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"), "-k", "not segment_struct_layout"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
