import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Print every parity comparison's error statistics (whole-tensor or
    sampled) at the end of the session, also under -q."""
    h = sys.modules.get("harness")
    if h is None or not getattr(h, "RESULTS", None):
        return
    terminalreporter.section("parity against the float64 oracle")
    for name, kind, res in h.RESULTS:
        vals = " ".join(f"{k}={v:.3e}" for k, v in res.items())
        terminalreporter.write_line(f"{name} [{kind}] {vals}")
