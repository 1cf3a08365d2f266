import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs a gfx950 GPU and the built HIP library")


def pytest_report_header(config):
    return "stream-K GEMM / wgrad engine tests (root %s)" % ROOT


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def no_fixup_timeouts(request):
    """Every GPU test must end with no hand-off wait given up: a wait that
    gives up folds nothing (its tile turns NaN) and is counted by the
    library; the count is zeroed before the test and checked after it.
    Tests that force give-ups on purpose reset the count themselves."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import implicit_gemm_conv_dp_amd as skg
    import torch
    torch.cuda.synchronize()
    skg.skg_fixup_timeouts(reset=True)
    yield
    torch.cuda.synchronize()
    n = skg.skg_fixup_timeouts(reset=True)
    assert n == 0, "%d hand-off waits gave up during the test" % n


def pytest_terminal_summary(terminalreporter):
    """Accuracy diagnostics of every tolerance comparison in the session:
    the infinity-norm relative error (the gate) and the element-wise
    relative error over |R| >= 2^-4 max |R|, worst case per input format."""
    try:
        from helpers import DIAGS
    except ImportError:
        return
    if not DIAGS:
        return
    tr = terminalreporter
    tr.write_sep("-", "accuracy diagnostics (tolerance comparisons)")
    for fmt in sorted({d[0] for d in DIAGS}):
        rows = [d for d in DIAGS if d[0] == fmt]
        wn = max(rows, key=lambda d: d[2])
        we = max(rows, key=lambda d: d[3])
        tr.write_line("%-5s %4d comparisons  max norm rel err %.3e (%s)  max elem rel err %.3e (%s)"
                      % (fmt, len(rows), wn[2], wn[1], we[3], we[1]))
