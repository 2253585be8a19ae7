"""The host side of the library and the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

libsq's C entry points (api.cpp, validate.cpp: every argument check, no HIP call) are compiled with
-fsanitize=address,undefined and linked with launcher stubs (tests/sanitize/host_launch_stubs.cpp); oracle.c is
compiled the same way. The ABI tests and the oracle's pins then run against these builds in a child process with
the sanitizer runtimes preloaded; any report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_transformer_attention_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _gcc_runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), r.stderr[-4000:])


def test_host_entry_points_and_oracle_are_clean_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's AddressSanitizer / UndefinedBehaviorSanitizer runtimes are not installed")
    lib = str(tmp_path / "libsq_host_san.so")
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "validate.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "host_launch_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(["g++", "-std=c++17", "-fPIC", "-Wall", "-I" + os.path.join(ROOT, "include")] + SAN + ["-c", src, "-o", obj])
        objs.append(obj)
    _run(["g++", "-shared", "-fPIC"] + SAN + objs + ["-o", lib])
    olib = str(tmp_path / "liboracle_san.so")
    _run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-Wall"] + SAN +
         [os.path.join(ROOT, "oracle", "oracle.c"), "-o", olib, "-lm"])
    env = dict(os.environ)
    env.update(SQ_LIBRARY=lib, SQ_ORACLE_LIBRARY=olib, LD_PRELOAD=asan + ":" + ubsan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in out
