import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle
    return _oracle.default()


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Every parity comparison of the session: normalised max error (the gate) and the 99.9th percentile of
    the elementwise relative error (reported only). ROM_PARITY_REPORT=<path> also writes them as JSON."""
    try:
        import parity
    except ImportError:
        return
    if not parity.REPORT:
        return
    tr = terminalreporter
    tr.section("parity errors (normalised max error | 99.9th-percentile elementwise relative error)")
    for label, name, err, p999, n in parity.REPORT:
        tr.write_line(f"{label:<44} {name:<13} {err:9.2e} | {p999:9.2e}  ({n} values)")
    path = os.environ.get("ROM_PARITY_REPORT")
    if path:
        parity.write_report(path)
