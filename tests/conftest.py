import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    return oracle


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    try:
        from ssd_testlib import ERRORS
    except ImportError:
        return
    if not ERRORS:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity: max|gpu - oracle| / max|oracle| over whole tensors")
    for label, ey, ef, tol in ERRORS:
        tr.write_line(f"{label:60s} y {ey:.3e}  final_states {ef:.3e}  (tol {tol:g}, "
                      f"margin {tol / max(ey, ef, 1e-30):.1f}x)")
