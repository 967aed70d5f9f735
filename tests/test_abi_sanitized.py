"""The C-ABI layer's host code under AddressSanitizer and UndefinedBehavior-
Sanitizer (CPU only, no GPU).

The library is rebuilt with both sanitizers on the host half of every source
(the gfx950 code is built as usual) into _build/sanitize/, and the host ABI
tests (tests/test_abi_host.py: every entry point's argument checks, malformed
shapes, NULL pointers, bad phase masks, short workspaces, malformed
cu_seqlens) run against it in a child process with the sanitizer runtime
preloaded.  Any report aborts the child, which fails this test."""
import glob
import os
import subprocess
import sys

import pytest

from block_sparse_backward_amd import build as lf_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT, "liblazyflash_sanitized.so")
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer", "-shared-libasan"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.slow
def test_abi_host_checks_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in /opt/rocm/llvm")
    lf_build.build(lib=LIB, objdir=OUT, host_flags=SANITIZE)
    log = os.path.join(OUT, "report")
    for f in glob.glob(log + ".*"):
        os.remove(f)
    env = dict(os.environ)
    env.update(LF_ABI_TEST_LIB=LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:faulthandler",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(log + ".*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], r.stderr[-3000:], reports[:4000])
