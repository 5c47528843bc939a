"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the library is rebuilt with host-only sanitizer flags
(w4a16_moe_decode_amd/_build_hostsan.py) and tests/test_abi.py runs against
it in a fresh interpreter with the sanitizer runtime preloaded.  Any report
aborts that process, so a clean exit with every test passed is the check."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_asan_ubsan():
    sys.path.insert(0, ROOT)
    from w4a16_moe_decode_amd import _build_hostsan
    lib = _build_hostsan.build()
    env = dict(os.environ)
    env.update({"LD_PRELOAD": _build_hostsan.runtime(), "FLINT_MOE_LIB": lib,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
