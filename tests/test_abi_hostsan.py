"""The host-side checks of the C ABI (tests/test_abi_host.py) run again against a build of the
library whose host code is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
(python -m delta_rule_sequence_amd.build --sanitize). CPU only: no kernel is launched, so the
argument checks, the sizing calls and the saved-buffer layout are what the sanitizers watch."""
import os
import subprocess
import sys

from delta_rule_sequence_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_checks_under_sanitizers():
    so = B.build(sanitize=True)
    undef = subprocess.run(["nm", "-D", "--undefined-only", so], stdout=subprocess.PIPE,
                           text=True, check=True).stdout
    assert "__asan_report" in undef and "__ubsan_handle" in undef, "host code not instrumented"
    preload = " ".join(p for p in (B.sanitizer_runtime(), os.environ.get("LD_PRELOAD", "")) if p)
    env = dict(os.environ, EFLA_LIBRARY_VARIANT="hostsan", LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    out = r.stdout
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out and "error" not in out.splitlines()[-1], out[-2000:]
