"""The host-side pool (pa_pool.cpp) under AddressSanitizer and UBSan, on the CPU.

pa_pool.cpp is built a second time with g++ and ``-fsanitize=address,undefined``
(no device code, so no GPU sanitizer is involved), then
  * the C client (tests/c_client.c) is linked against that build and run, with
    leak checking on;
  * the pool's parity tests (test_alloc_parity.py, test_shared_groups.py) run
    in a child pytest whose pool calls go to that build (tests/san_plugin.py),
    with the ASan runtime preloaded.
Any sanitizer report fails the run (``-fno-sanitize-recover=all``, non-zero
exit on a report).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POOL_SRC = os.path.join(ROOT, "paged_kv_cache_06_amd", "csrc", "pa_pool.cpp")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _runtime(cxx, name):
    out = subprocess.run([cxx, f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def toolchain():
    cxx, cc = shutil.which("g++"), shutil.which("gcc")
    if cxx is None or cc is None:
        pytest.skip("no gcc/g++")
    asan = _runtime(cxx, "libasan.so")
    if asan is None:
        pytest.skip("no ASan runtime")
    return cxx, cc, asan


def _env(**extra):
    env = dict(os.environ)
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def test_c_client_under_asan_and_ubsan(toolchain, tmp_path):
    cxx, cc, _ = toolchain
    inc = os.path.join(ROOT, "include")
    obj = tmp_path / "c_client.o"
    exe = tmp_path / "c_client_san"
    steps = [
        [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", *SAN, "-I", inc, "-c",
         os.path.join(ROOT, "tests", "c_client.c"), "-o", str(obj)],
        [cxx, "-std=c++17", "-Wall", "-Wextra", "-Werror", *SAN, "-I", inc, str(obj), POOL_SRC,
         "-o", str(exe)],
    ]
    for cmd in steps:
        built = subprocess.run(cmd, capture_output=True, text=True)
        assert built.returncode == 0, built.stderr
    ran = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120,
                         env=_env(ASAN_OPTIONS="detect_leaks=1:halt_on_error=1"))
    assert ran.returncode == 0, ran.stdout[-2000:] + ran.stderr[-4000:]
    assert "0 failure(s)" in ran.stdout
    assert "runtime error" not in ran.stderr and "AddressSanitizer" not in ran.stderr


@pytest.mark.slow
def test_pool_parity_tests_under_asan_and_ubsan(toolchain, tmp_path):
    cxx, _, asan = toolchain
    lib = tmp_path / "libpa_pool_san.so"
    cmd = [cxx, "-std=c++17", "-Wall", "-Wextra", "-Werror", *SAN, "-shared", "-fPIC", "-I",
           os.path.join(ROOT, "include"), POOL_SRC, "-o", str(lib)]
    built = subprocess.run(cmd, capture_output=True, text=True)
    assert built.returncode == 0, built.stderr
    # leaks are not checked here: the interpreter itself holds memory at exit
    env = _env(LD_PRELOAD=asan, PA_SAN_POOL_LIB=str(lib),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    ran = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-s", "-p", "tests.san_plugin", "-p", "no:cacheprovider",
         "-m", "not gpu", os.path.join("tests", "test_alloc_parity.py"),
         os.path.join("tests", "test_shared_groups.py")],
        cwd=ROOT, capture_output=True, text=True, timeout=900, env=env)
    assert ran.returncode == 0, ran.stdout[-3000:] + ran.stderr[-4000:]
    assert " passed" in ran.stdout and "failed" not in ran.stdout
    assert "runtime error" not in ran.stderr and "AddressSanitizer" not in ran.stderr
