import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the figures the tests reported (error metrics at full size, drift
    curves, whole-stack latency and memory) after the test summary."""
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    if tests_dir not in sys.path:
        sys.path.insert(0, tests_dir)
    import helpers
    if helpers.REPORT:
        terminalreporter.section("gdn parity report")
        for line in helpers.REPORT:
            terminalreporter.write_line(line)
