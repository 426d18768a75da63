"""The CPU oracle and the library's host side (the C ABI's argument checks, with launchers
that launch nothing) built under AddressSanitizer and UndefinedBehaviorSanitizer, and the
oracle, ABI and host-contract tests run against those builds in a child process (the
sanitizer runtime has to be preloaded into an uninstrumented Python). Any finding aborts
the child. A planted overflow and a planted signed overflow, in a throwaway library of
this test, show that the harness does catch both kinds."""
import os
import shutil
import subprocess
import sys

import pytest

from bit_kv_cache_pack_amd import build as KB
from oracle import build_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECKED_TESTS = ["tests/test_abi_host.py", "tests/test_host_contract.py",
                 "tests/test_oracle_quant.py", "tests/test_oracle_attention.py",
                 "tests/test_oracle_paged.py", "tests/test_oracle_keynorm.py",
                 "tests/test_oracle_outer.py"]


def _asan_runtime():
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("no host compiler")
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                       text=True).stdout.strip()
    if not p or not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("no AddressSanitizer runtime")
    return p


def _env(asan, **extra):
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1")
    env.update(extra)
    return env


def test_harness_catches_planted_errors(tmp_path):
    asan = _asan_runtime()
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int overflow(int n) { int *a = malloc(4 * n); a[n] = 1; int r = a[0]; "
                   "free(a); return r; }\n"
                   "int add(int a, int b) { return a + b; }\n")
    lib = tmp_path / "libplanted.so"
    subprocess.run(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", str(lib), str(src)], check=True)
    for call, marker in (("overflow(4)", "heap-buffer-overflow"),
                         ("add(2147483647, 1)", "signed integer overflow")):
        code = (f"import ctypes; L = ctypes.CDLL({str(lib)!r}); "
                f"L.{call.split('(')[0]}.argtypes = [ctypes.c_int] * "
                f"{call.count(',') + 1}; L.{call}")
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                           env=_env(asan), timeout=120)
        assert r.returncode != 0 and marker in r.stderr, (call, r.returncode, r.stderr[-500:])


def test_oracle_and_host_checks_clean_under_sanitizers(tmp_path):
    asan = _asan_runtime()
    host = KB.build_host_checked(str(tmp_path / "libkvq_host_checked.so"))
    orc = build_oracle.build(sanitize=True, out=str(tmp_path / "liboracle_checked.so"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu and not slow", *CHECKED_TESTS],
                       cwd=ROOT, capture_output=True, text=True, timeout=900,
                       env=_env(asan, KVQ_LIB_PATH=host, KVQ_ORACLE_LIB_PATH=orc))
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail
