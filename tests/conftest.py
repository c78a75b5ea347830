import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")
    config.addinivalue_line("markers", "slow: long-running")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Per-case parity figures of the GPU tests (max |out - ref| / max |ref| over the checked tokens
    against the oracle), printed after the run even when output capture hides the tests' own lines."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    try:
        import moe_testlib
    except Exception:  # the CPU-only suite may not import it
        return
    if not moe_testlib.RESULTS:
        return
    terminalreporter.write_sep("-", "parity against the oracle: max|out-ref| / max|ref| (checked tokens, flagged)")
    for label, rel, n, flagged in moe_testlib.RESULTS:
        terminalreporter.write_line("%-40s %.3e  tokens %6d  flagged %d" % (label, rel, n, flagged))
