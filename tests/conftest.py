import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

import parity_log  # noqa: E402


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Worst GPU-vs-oracle errors of the session, per group (the five
    workloads c1..c5 by name; other shapes by their label's first word), so
    that a quiet run's record holds the error magnitudes."""
    recs = parity_log.RECORDS
    if not recs:
        return
    groups = {}
    for what, rel, mx in recs:
        g = parity_log.group_of(what)
        n, r0, m0 = groups.get(g, (0, 0.0, 0.0))
        groups[g] = (n + 1, max(r0, rel), max(m0, mx))
    tr = terminalreporter
    worst_rel = max(r for _, r, _ in recs)
    worst_mx = max(m for _, _, m in recs)
    tr.write_line(f"parity vs oracle: {len(recs)} comparisons, worst rel_l2 {worst_rel:.2e} (bar 1e-5), "
                  f"worst max_abs/max|ref| {worst_mx:.2e} (bar 1e-4)")
    keys = sorted(groups, key=lambda k: (not (len(k) == 2 and k[0] == "c"), k))
    line = []
    for k in keys:
        n, r, m = groups[k]
        line.append(f"{k}: n={n} rel {r:.1e} max {m:.1e}")
        if len(line) == 3:
            tr.write_line("  " + " | ".join(line))
            line = []
    if line:
        tr.write_line("  " + " | ".join(line))
