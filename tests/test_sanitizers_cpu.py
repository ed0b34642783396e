"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only, no device is touched):

* the oracle (oracle.c) built by gcc with both sanitizers, every pin run
  against it in a process whose first library is gcc's libasan;
* the C-ABI layer of the library (argument validation, planning, workspace
  layout, tuning table, plan overrides, the static scratch's size check)
  compiled with both sanitizers on the host side by hipcc, then the C99 ABI
  program and tests/test_abi_cpu.py run against that build in processes whose
  first library is clang's ASan runtime.

Any report from either sanitizer makes the process fail (UBSan does not
recover; ASan aborts on its first error).  Leak checking is off: the Python
interpreter and the HIP runtime keep allocations for the process lifetime.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_OPTIONS = "detect_leaks=0:abort_on_error=1:detect_odr_violation=0:alloc_dealloc_mismatch=0"


def _gcc_libasan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run(code_or_args, env_extra, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS=ASAN_OPTIONS, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=os.pathsep.join([ROOT, os.path.join(ROOT, "tests")]), **env_extra)
    args = code_or_args if isinstance(code_or_args, list) else [sys.executable, "-c", code_or_args]
    return subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


@pytest.mark.skipif(shutil.which("gcc") is None or _gcc_libasan() is None, reason="needs gcc with libasan")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    code = ("import oracle, oracle_pins\n"
            f"with oracle.using({lib!r}):\n"
            "    for pin in oracle_pins.ALL_PINS:\n"
            "        pin()\n"
            "print('pins ok', len(oracle_pins.ALL_PINS))\n")
    res = _run(code, {"LD_PRELOAD": _gcc_libasan(), "OMP_NUM_THREADS": "4"})
    assert res.returncode == 0 and "pins ok" in res.stdout, res.stdout[-3000:] + res.stderr[-6000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-6000:]


@pytest.fixture(scope="module")
def sanitized_library(tmp_path_factory):
    if shutil.which("/opt/rocm/bin/hipcc") is None or _clang_asan() is None:
        pytest.skip("needs hipcc and clang's ASan runtime")
    from fusion_residual_add_amd import build
    return build.build_host_sanitized(str(tmp_path_factory.mktemp("san") / "libfusedproj_san.so"))


def test_c_abi_program_under_asan_ubsan(sanitized_library, tmp_path):
    clang = "/opt/rocm/lib/llvm/bin/clang"
    exe = str(tmp_path / "abi_check_san")
    libdir = os.path.dirname(sanitized_library)
    link = os.path.join(libdir, "libfusedproj.so")
    if not os.path.exists(link):
        os.symlink(sanitized_library, link)
    subprocess.run([clang, "-std=c99", "-Wall", "-Werror", "-pedantic", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-shared-libsan", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", libdir, "-lfusedproj",
                    "-Wl,-rpath," + libdir, "-Wl,-rpath," + os.path.dirname(_clang_asan()), "-o", exe],
                   check=True, capture_output=True, text=True)
    res = _run([exe], {})
    assert res.returncode == 0 and "abi_check ok" in res.stdout, res.stdout[-3000:] + res.stderr[-6000:]


def test_abi_tests_under_asan_ubsan(sanitized_library):
    res = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                os.path.join(ROOT, "tests", "test_abi_cpu.py")],
               {"LD_PRELOAD": _clang_asan(), "FUSEDPROJ_LIBRARY": sanitized_library}, timeout=900)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-6000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-6000:]
