"""CPU checks under AddressSanitizer and UndefinedBehaviorSanitizer.

Two builds of this repository's C and host C++ code, made in a temporary
directory for these tests only:
  * the oracle (plain C) with -fsanitize=address,undefined, against which
    tests/test_oracle_pins.py runs in full;
  * the C-ABI library with the sanitizers on its host code only (the device
    code is built as usual), against which tests/test_abi_cpu.py runs: every
    argument check of every entry point, no device work.
A planted out-of-bounds read in a copy of the oracle shows that the
sanitizer is live.  Each run is a subprocess with the sanitizer runtime of
its compiler preloaded (gcc's for the oracle, the ROCm clang's for the
library).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "bitlinear_oracle.c")
CSRC = os.path.join(ROOT, "bitlinear_quant_act_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "4"}


def _gcc_runtime(name):
    return subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True,
                          check=True).stdout.strip()


def _build_oracle(src_text, out):
    c = out + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
                    "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", c, "-o", out, "-lm"], check=True)


def _run_pins(lib, log_dir=None):
    env = dict(os.environ, BITLINEAR_ORACLE_LIB=lib, **SAN_ENV,
               LD_PRELOAD=_gcc_runtime("libasan.so") + " " + _gcc_runtime("libubsan.so"))
    if log_dir is not None:  # the report goes to a file: pytest's capture would swallow it
        env["ASAN_OPTIONS"] += ":log_path=" + os.path.join(log_dir, "asan")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_oracle_pins_under_sanitizers(tmp_path):
    with open(ORACLE_SRC) as f:
        src = f.read()
    lib = str(tmp_path / "liboracle_san.so")
    _build_oracle(src, lib)
    r = _run_pins(lib)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_sanitizer_reports_a_planted_overflow(tmp_path):
    """A copy of the oracle reading one value past each token's row must be
    stopped by AddressSanitizer (heap-buffer-overflow on the last token)."""
    with open(ORACLE_SRC) as f:
        src = f.read()
    old = "            float v = fabsf(bf16_to_f32(x[r * k + c]));"
    assert src.count(old) == 1
    lib = str(tmp_path / "liboracle_planted.so")
    _build_oracle(src.replace(old, "            float v = fabsf(bf16_to_f32(x[r * k + c + 1]));"), lib)
    r = _run_pins(lib, str(tmp_path))
    assert r.returncode != 0
    reports = "".join(open(f).read() for f in glob.glob(str(tmp_path / "asan*")))
    assert "heap-buffer-overflow" in reports, reports[-2000:]


def test_abi_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not runtimes:
        pytest.skip("the ROCm clang sanitizer runtime is not installed")
    # sanitizers on the host side of every source only (each -fsanitize is
    # scoped to the host compilation); the device code is built as usual
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-fast-math", "-ffp-contract=off",
             "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + host_san
    procs, objs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", src, "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT))
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out[-2000:]
    lib = str(tmp_path / "libbitlinear_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", *objs, "-o", lib], check=True)
    env = dict(os.environ, BITLINEAR_TEST_LIB=lib, LD_PRELOAD=runtimes[0], **SAN_ENV)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
