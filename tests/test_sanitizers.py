"""Sanitizer runs on the CPU (AddressSanitizer + UndefinedBehaviorSanitizer).

1. The oracle, built with -fsanitize=address,undefined (undefined behaviour fatal), runs its
   whole pin suite in a child process (libasan preloaded into the interpreter).
2. The library's host code -- configuration checks, level progression, parameter layout,
   workspace plans of every entry point and the argument checks -- built with the sanitizers
   on the host side only, runs the driver in tests/sanitize/host_driver.c, which queries
   sizes and hands every compute entry point arguments it must reject before launching (no
   GPU is touched).
"""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "multiresolution_hash_grid_multires_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name):
    try:
        path = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def pin_files():
    from tests.test_pins_mutations import pin_files as files
    return files()


def _instrumented(path):
    out = subprocess.run(["nm", "-D", path], capture_output=True, text=True).stdout
    return "__asan_init" in out or "__asan_report_load4" in out


def test_oracle_pins_under_sanitizers(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    from oracle.oracle import build_oracle
    lib = build_oracle(out=str(tmp_path / "liboracle_san.so"),
                       extra_flags=["-O1", "-g", "-fsanitize=address,undefined",
                                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"])
    assert _instrumented(lib)
    tests = pin_files()
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=f"{asan}:{ubsan}", HASHGRID_ORACLE_LIB=lib,
               OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout


def test_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    flags = ["--offload-arch=gfx950", "-O1", "-Xarch_device", "-O0", "-g", "-std=c++20",
             "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer", f"-I{INCLUDE}", f"-I{CSRC}"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.check_call([HIPCC, *flags, "-c", src, "-o", obj], stderr=subprocess.DEVNULL)
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        objs = list(pool.map(compile_one, srcs))
    exe = str(tmp_path / "host_driver")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address,undefined",
                           f"-I{INCLUDE}", "-x", "c++", os.path.join(ROOT, "tests", "sanitize", "host_driver.c"),
                           "-x", "none", *objs, "-o", exe], stderr=subprocess.DEVNULL)
    syms = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    r = subprocess.run([exe], env=dict(os.environ, **SAN_ENV), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "all expectations met" in r.stdout
    shutil.rmtree(tmp_path, ignore_errors=True)
