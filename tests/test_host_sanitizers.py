"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

Every library source is compiled with both sanitizers on the host pass only
(the device code is built as usual and never launched here: every call
fails validation first), and linked into a temporary copy of the library.
tests/test_abi.py then runs against that copy in a child process with the
sanitizer runtime preloaded (HNA_LIB_PATH selects the copy); any report
aborts the child and fails this test.  Leak checking is off: the interpreter itself keeps allocations alive
until exit.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from head_neuron_affinity_amd import build_lib as B  # noqa: E402

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    r = subprocess.run([B.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(900)
def test_abi_validation_clean_under_asan_and_ubsan(tmp_path):
    rt = _runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    objs, jobs = [], []
    for src in B.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([B.HIPCC, *B.FLAGS, "-g", *SAN, *B.EXTRA.get(src, []),
                     "-c", os.path.join(B.CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=4) as ex:
        for r in ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), jobs):
            assert r.returncode == 0, r.stderr[-3000:]
    lib = str(tmp_path / "libhna.so")
    r = subprocess.run([B.HIPCC, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *SAN, *objs,
                        "-o", lib, *B.LIBS],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the copy is instrumented: it calls into both runtimes
    und = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in und and "__ubsan_handle" in und

    env = dict(os.environ)
    env.update(HNA_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0:"
                            "alloc_dealloc_mismatch=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
    assert " passed" in r.stdout, out
