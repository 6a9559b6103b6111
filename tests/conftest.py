import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per parity case: the largest error of each stage and its
    share of the gate (q_lat, q_pe, o_lat, o row-normwise; lse absolute)."""
    from tests._metrics import RECORDED

    if not RECORDED:
        return
    tr = terminalreporter
    tr.section("parity margins (max error per stage / gate)")
    worst = 0.0
    for label, errs, tol in RECORDED:
        frac = max(errs.values()) / tol if errs else 0.0
        worst = max(worst, frac)
        tr.write_line(f"{label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items())
                      + f" gate={tol:.2g} worst={frac:.2f}")
    tr.write_line(f"{len(RECORDED)} cases, largest error / gate = {worst:.2f}")
