"""The GPU parity tests again, in a child process, against the LDS-poison build of the library
(libefla_ldspoison.so, built by python -m delta_rule_sequence_amd.build --lds-poison): there every
kernel fills its dynamic LDS with all-ones bytes (NaN in fp32 and bf16) before it starts. A kernel
that reads an LDS location it has not written in the same launch (a partial chunk's rows, padding,
a tile the loader has not filled yet) then produces NaN, which the parity tests reject, where the
normal build would read stale values that may happen to be harmless.

The child's output goes straight to this process's stdout, one line per test."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POISON_SO = os.path.join(ROOT, "delta_rule_sequence_amd", "libefla_ldspoison.so")
FILES = ["test_gpu_parity.py", "test_gpu_wide_ragged.py", "test_gpu_segments.py",
         "test_gpu_gated.py", "test_gpu_state_modes.py"]


@pytest.mark.timeout(1500)
def test_parity_suite_with_poisoned_lds():
    assert os.path.exists(POISON_SO), \
        "libefla_ldspoison.so is not built: python -m delta_rule_sequence_amd.build --lds-poison"
    env = dict(os.environ, EFLA_LIBRARY_VARIANT="ldspoison")
    cmd = [sys.executable, "-u", "-m", "pytest", "-x", "-v", "-m", "gpu", "-p", "no:cacheprovider",
           "--timeout", "300", "--timeout-method", "thread"]
    cmd += [os.path.join(ROOT, "tests", f) for f in FILES]
    print("LDS-poison build: running", " ".join(FILES), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, env=env, timeout=1450)
    assert r.returncode == 0, "parity failed with poisoned LDS (exit status %d)" % r.returncode
