"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two builds, each run in a child process with its sanitizer runtime preloaded
(Python itself is not instrumented):
  * libretention's host code (argument validation, overlap and size checks,
    planning, the plan override) built with clang's ASan + UBSan
    (retention_chunkwise_amd._build --sanitize-host; device code unchanged),
    driven by tests/test_abi.py;
  * the fp64 oracle built with gcc's ASan + UBSan, driven by its pins and the
    parity-metric pins.
Any out-of-bounds access, use after free or undefined behaviour aborts the
child, and the test fails with its report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(code, preload, timeout=900):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    print(tail)
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail


def test_library_host_code_under_asan_ubsan():
    from retention_chunkwise_amd import _build

    try:
        lib = _build.build(sanitize_host=True)  # incremental: objects kept under _build/asan
        rt = _build.asan_runtime()
    except RuntimeError as e:  # pragma: no cover - no ROCm toolchain
        pytest.skip(f"cannot build the sanitized library: {e}")
    code = ("import sys, pytest, retention_chunkwise_amd as rc\n"
            f"rc._LIB_PATH = {lib!r}\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_abi.py']))\n")
    _child(code, rt)


def test_oracle_under_asan_ubsan(tmp_path):
    src = os.path.join(ROOT, "oracle", "oracle.c")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", lib, src, "-lm"],
                   check=True)
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    code = ("import sys, pytest, oracle\n"
            f"with oracle.using_library({lib!r}):\n"
            "    rc = pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_oracle_pins.py',"
            " 'tests/test_metric_pins.py'])\n"
            "sys.exit(rc)\n")
    _child(code, rt)
