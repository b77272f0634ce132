import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the error margins the full-size parity checks recorded (tolerances: rel-L2 5e-3,
    max-abs 2e-2 of max|ref|), so that a quiet run still records them."""
    import parity

    if not parity.MARGINS:
        return
    terminalreporter.section("parity margins (rel-L2 <= 5e-3, max-abs/max|ref| <= 2e-2)")
    for what, rel, mx in parity.MARGINS:
        terminalreporter.write_line(f"{what}: rel-L2 {rel:.3e}, max-abs/max|ref| {mx:.3e}")
