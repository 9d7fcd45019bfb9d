"""CPU sanitizer runs (no GPU): the oracle built with AddressSanitizer and
UndefinedBehaviorSanitizer runs every oracle pin, and the library's host code
(argument validation, workspace carving, launch set-up in abi.hip) built with
the same sanitizers on its host side runs the C-ABI validation cases. Each run
is a child process with the sanitizer runtime preloaded; any report fails it.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, env_extra):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_pins_under_asan_ubsan():
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "libmoe_oracle_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
                        "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-shared", "-fPIC",
                        os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", lib, "-lm"],
                       check=True)
        out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                    "tests/test_oracle_pins.py", "tests/test_oracle_exact_layer.py"],
                   {"LD_PRELOAD": libasan, "MOE_ORACLE_LIB": lib})
    assert " passed" in out


def test_abi_host_code_under_asan_ubsan():
    from w8a8_int8_expert_amd import build
    hipcc = build._hipcc()
    rt = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt):
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    objs = sorted(os.path.join(build.BUILD, f) for f in os.listdir(build.BUILD)
                  if f.endswith(".o") and f != "abi.o") if os.path.isdir(build.BUILD) else []
    if len(objs) < 5:
        build.build()
        objs = sorted(os.path.join(build.BUILD, f) for f in os.listdir(build.BUILD)
                      if f.endswith(".o") and f != "abi.o")
    with tempfile.TemporaryDirectory() as d:
        obj = os.path.join(d, "abi_san.o")
        lib = os.path.join(d, "libmoe_w8a8_san.so")
        # host side only: the device code of abi.hip is not instrumented
        flags = [f for f in build.compile_flags()]
        subprocess.run([hipcc, "-c", os.path.join(build.CSRC, "abi.hip"), "-o", obj] + flags +
                       ["-g", "-fno-omit-frame-pointer",
                        "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=undefined"],
                       check=True, capture_output=True)
        subprocess.run([hipcc, "-shared", "--offload-arch=" + build.ARCH, "-o", lib, obj] + objs +
                       ["-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"],
                       check=True, capture_output=True)
        out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                    "tests/test_abi_cpu.py"],
                   {"LD_PRELOAD": rt, "MOE_W8A8_TEST_LIB": lib})
    assert " passed" in out
