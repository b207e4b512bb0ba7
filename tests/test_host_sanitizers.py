"""The C ABI tests (host-side checks, workspace queries, CG and template
tables, the binding's guards) run against a build of the library whose host
code carries AddressSanitizer and UndefinedBehaviorSanitizer, every finding
fatal.  CPU only: the sanitized build launches no kernel."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_asan_and_ubsan():
    # imported here: the build script is host tooling that GPU runs do not carry
    from equivariant_gnn_electronic_amd import build_sanitized as bs
    lib = bs.build_if_stale()
    # PYTHONMALLOC=malloc: the interpreter's own buffers come from the sanitizer's allocator too
    env = dict(os.environ, EGNN_LIBRARY=lib, LD_PRELOAD=bs.asan_runtime(), PYTHONMALLOC="malloc",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    last = r.stdout.strip().splitlines()[-1]
    assert "passed" in last and "failed" not in last and "error" not in last, last
