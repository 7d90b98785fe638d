import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter):
    from tests import parity_log

    if parity_log.LINES:
        terminalreporter.section("whole-workload parity (max-abs and mean-abs error against the oracle)")
        for line in parity_log.LINES:
            terminalreporter.write_line(line)
