"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

1. The oracle (plain C, gcc) linked into tests/sanitize/oracle_checks.c, which calls every
   exported oracle function on small seeded problems of the shapes the parity tests use, with
   every option bit, and the arguments each call must reject.
2. The library (hipcc, the instrumentation on the host pass only; the device code is built as
   usual and never runs here) with tests/sanitize/abi_checks.c, which drives every C-ABI entry
   point through the argument validation that runs before any device call, the workspace-size
   queries over a range of shapes, and the status strings.

Each test passes when its driver exits 0 and the sanitizers report nothing.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE = os.path.join(ROOT, "oracle")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout, r.stderr


def _assert_clean(rc, out, err, ok_line):
    assert rc == 0, f"driver exit status {rc}\n{out}\n{err[-4000:]}"
    assert ok_line in out
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in err, err[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", ORACLE, os.path.join(SAN, "oracle_checks.c"),
           os.path.join(ORACLE, "sage_oracle.c"), os.path.join(ORACLE, "sagebwd_oracle.c"), "-lm", "-o", exe]
    rc, out, err = _run(cmd)
    assert rc == 0, err[-4000:]
    _assert_clean(*_run([exe], env=ENV, timeout=600), "oracle checks ok")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_library_host_code_under_asan_ubsan(tmp_path):
    from quantized_attention_amd import build as b

    # the library's own flags; the instrumentation and debug info apply to the host pass only
    # (each sanitizer flag sits right after -Xarch_host), the device code is built as usual
    flags = [*b.FLAGS, "-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]

    def one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        rc, _, err = _run([HIPCC, *flags, "-c", src, "-o", obj])
        assert rc == 0, err[-4000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, b.sources()))
    lib = str(tmp_path / "libsage_san.so")
    rc, _, err = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                       "-Xarch_host", "-fsanitize=undefined", *objs, "-o", lib])
    assert rc == 0, err[-4000:]
    exe = str(tmp_path / "abi_checks")
    rc, _, err = _run(["/opt/rocm/llvm/bin/clang", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                       "-I", b.INCLUDE, os.path.join(SAN, "abi_checks.c"), lib, "-o", exe,
                       f"-Wl,-rpath,{tmp_path}"])
    assert rc == 0, err[-4000:]
    _assert_clean(*_run([exe], env=ENV, timeout=300), "abi checks ok")
