"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds, into a temporary directory, libmla.so with its host code
instrumented (the device code is built as usual; on this toolchain the
sanitizers apply to host code only) and the C oracle instrumented, then
runs the CPU test files that exercise them (argument checks of every entry
point, the host audit fed bad tables, the oracle, its pins and the
schedule) in a child process with the sanitizer runtime preloaded.  Any
sanitizer report fails the run (UBSan is fatal on its first error)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CPU_FILES = ["tests/test_abi.py", "tests/test_host_audit.py", "tests/test_oracle.py", "tests/test_codec.py",
             "tests/test_schedule.py", "tests/test_kv_append_oracle.py"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_cpu_suite_clean_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no clang sanitizer runtime / hipcc in this image")
    from mla_paged_kv_metadata_amd import build as B
    lib = B.build(extra=["-O1", "-g", "-fno-omit-frame-pointer",
                         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                         "-Xarch_host", "-fno-sanitize-recover=undefined"],
                  out=str(tmp_path / "libmla_san.so"), objdir=str(tmp_path / "obj"),
                  link_extra=["-shared-libsan", "-Xarch_host", "-fsanitize=address",
                              "-Xarch_host", "-fsanitize=undefined"])
    orc = str(tmp_path / "liboracle_san.so")
    subprocess.run(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
                    "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", "-o", orc,
                    os.path.join(ROOT, "oracle", "mla_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=rt, MLA_LIB_PATH=lib, MLA_ORACLE_LIB=orc,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *CPU_FILES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
