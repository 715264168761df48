import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter):
    """Margins of the floating-point parity compares: per test, the largest fraction of
    the allowed error (atol + rtol*|ref|) any compared element used, with max-abs and
    max-rel errors."""
    mod = sys.modules.get("tests.gpu_util")
    rows = getattr(mod, "MARGINS", None) if mod else None
    if not rows:
        return
    worst = {}
    for test, what, dt, ma, mr, fr in rows:
        k = (test, what, dt)
        if k not in worst or fr > worst[k][2]:
            worst[k] = (ma, mr, fr)
    tr = terminalreporter
    tr.write_sep("-", "parity margins (%d compares)" % len(rows))
    for (test, what, dt), (ma, mr, fr) in sorted(worst.items(), key=lambda kv: -kv[1][2])[:40]:
        tr.write_line("%.3f of allowed  max abs %.3g  max rel %.3g  %s  %s  %s" % (fr, ma, mr, dt, what, test))
