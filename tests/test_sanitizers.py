"""The host-side tests (oracle pins, C ABI checks) rerun under
AddressSanitizer and UBSan: the oracle and the host side of the C ABI are
rebuilt with both (clang, shared sanitizer runtime) and a child pytest loads
them, with the runtime preloaded into the interpreter.  Any report fails the
child (UBSan without recovery; ASan aborts on the first error)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def test_host_tests_under_address_and_undefined_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's shared AddressSanitizer runtime is not available")
    sys.path.insert(0, ROOT)
    import oracle
    from fp4_block_scaled_row_amd import build
    if not os.path.exists(os.path.join(build.BUILD_DIR, "fp4q_mx.o")):
        pytest.skip("the HIP library is not built (run __graft_entry__.build())")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               FP4Q_ORACLE_LIB=oracle.build_sanitized(), FP4Q_LIB=build.build_sanitized_host())
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
