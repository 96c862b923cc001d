"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

(1) The fp64 oracle (oracle/gdn_oracle.c), built by gcc with -fsanitize=address,undefined
    (no recovery), runs every oracle pin (tests/test_oracle_pins.py) in a child process with the
    sanitizer runtime preloaded.
(2) The C ABI's host side (csrc/gdn_api.hip: argument validation, workspace sizes, plans, the
    no-allocation entry point's size check), built by hipcc with the sanitizers on the host pass
    only and linked with the other objects of the library, runs the ABI tests
    (tests/test_abi_cpu.py), none of which reaches a kernel.
A sanitizer report makes the child exit non-zero.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_tests(test_file, env_extra, tmp_path):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", test_file), "-q", "-x",
           "-m", "not gpu", "-p", "no:cacheprovider"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    log = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, log
    assert "ERROR: AddressSanitizer" not in log and "runtime error" not in log, log
    return log


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libgdn_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-o", lib, os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True,
                           text=True, check=True).stdout.strip()
    log = _run_tests("test_oracle_pins.py", {"GDN_ORACLE_LIB": lib,
                                             "LD_PRELOAD": asan + ":" + ubsan}, tmp_path)
    assert " passed" in log


def test_abi_host_side_under_asan_ubsan(tmp_path):
    build = os.path.join(ROOT, "linear_attention_token_gdn_amd", "_build")
    csrc = os.path.join(ROOT, "linear_attention_token_gdn_amd", "csrc")
    others = [os.path.join(build, n + ".o") for n in
              ("decode", "recurrent", "chunk_mfma", "chunk_split", "backward", "backward_chunk",
               "qsa")]
    if not all(os.path.exists(p) for p in others):
        from linear_attention_token_gdn_amd import build as hipbuild
        hipbuild.build()
    rt = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm installation")
    obj, lib = str(tmp_path / "gdn_api_san.o"), str(tmp_path / "libgdn_san.so")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
                    "-c", os.path.join(csrc, "gdn_api.hip"), "-o", obj], check=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, obj, *others],
                   check=True)
    log = _run_tests("test_abi_cpu.py", {"GDN_LIBRARY": lib, "LD_PRELOAD": rt[0]}, tmp_path)
    assert " passed" in log
