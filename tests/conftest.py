import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle runs that take more than a few seconds")


def pytest_report_header(config):
    if os.environ.get("EFLA_LIBRARY_VARIANT"):
        from delta_rule_sequence_amd import _lib
        return "EFLA library variant: %s" % _lib.LIB_PATH
