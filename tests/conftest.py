import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Parity margins of the layer-output checks, (label, rel_l2, max_abs/rms),
# appended by the GPU parity tests and printed at the end of the run, so the
# margin of every case reaches the run's record and not only its pass/fail.
PARITY_LOG = []


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if not PARITY_LOG:
        return
    tr = terminalreporter
    tr.section("parity margins (bars: rel_l2 <= 5e-3, max_abs <= 2e-2 * rms)")
    worst_rel = max(r for _, r, _ in PARITY_LOG)
    worst_abs = max(m for _, _, m in PARITY_LOG)
    for label, rel, mx in PARITY_LOG:
        tr.write_line(f"{label:60s} rel_l2={rel:.2e} ({5e-3 / rel:6.1f}x inside)  "
                      f"max_abs/rms={mx:.2e} ({2e-2 / mx:6.1f}x inside)")
    tr.write_line(f"worst: rel_l2 {worst_rel:.2e} ({5e-3 / worst_rel:.1f}x inside), "
                  f"max_abs/rms {worst_abs:.2e} ({2e-2 / worst_abs:.1f}x inside), {len(PARITY_LOG)} checks")
