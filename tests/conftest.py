import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


def pytest_terminal_summary(terminalreporter):
    """The parity checks' worst-chunk and final-weight errors, one line each."""
    pc = sys.modules.get("parity_check")
    lines = getattr(pc, "REPORT", None) if pc else None
    if lines:
        terminalreporter.section("parity errors against the oracle (worst chunk per check)")
        for line in lines:
            terminalreporter.write_line(line)
