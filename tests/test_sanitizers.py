"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU oracle and of
libisg's host layer, each driven by the existing CPU tests in a child process.

* The oracle (gcc, -fsanitize=address,undefined) runs every oracle pin, so each
  oracle function is exercised on the pins' inputs.
* libisg is built with the sanitizers on its host code only (device code as
  usual) and runs the C-ABI checks: library load, exports, workspace sizes, the
  proposal table and every argument-validation path.  No kernel is launched.

UBSan stops at the first finding (-fno-sanitize-recover), ASan at its first
report; leak checking is off because the Python interpreter itself keeps memory
until exit.  The child's exit status and output decide the test.
"""
import glob
import importlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ENV_BASE = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan():
    if not shutil.which("gcc"):
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _undefined_asan_symbols(lib):
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    return [l for l in out.splitlines() if "__asan_report" in l or "__ubsan_handle" in l]


def _run_child(test_file, env_extra, preload):
    env = dict(os.environ, **ENV_BASE, **env_extra, LD_PRELOAD=preload)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", test_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    return r.returncode, out


def test_oracle_under_asan_ubsan():
    rt = _gcc_asan()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = importlib.import_module("oracle.build").build(sanitize=True)
    assert _undefined_asan_symbols(lib), "the oracle build is not instrumented"
    rc, out = _run_child("test_oracle_pins.py", {"ISG_ORACLE_LIB": lib}, rt)
    tail = "\n".join(out.splitlines()[-30:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, tail
    assert rc == 0 and " passed" in out, tail


def test_abi_host_layer_under_asan_ubsan():
    rt = _clang_asan()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    lib = importlib.import_module("block_sparse_attention_means_amd.csrc.build").build(sanitize=True)
    assert _undefined_asan_symbols(lib), "the host build is not instrumented"
    rc, out = _run_child("test_abi_cpu.py", {"ISG_LIBRARY": lib}, rt)
    tail = "\n".join(out.splitlines()[-30:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, tail
    assert rc == 0 and " passed" in out, tail
