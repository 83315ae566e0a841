import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter):
    helpers = sys.modules.get("gpu_helpers")
    lines = getattr(helpers, "SUMMARY", None)
    if lines:
        terminalreporter.section("greedy parity")
        for line in lines:
            terminalreporter.write_line(line)


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    from oracle import build
    build.build(force=False)
    return oracle
