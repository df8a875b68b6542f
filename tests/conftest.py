import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (multi-GB inputs)")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Report the routing flips (certified near-ties between the GPU's and the oracle's own float32
    router logits) of every end-to-end parity case that ran."""
    try:
        import parity
    except Exception:   # the CPU-only suite may not have imported it
        return
    log = getattr(parity, "FLIP_LOG", [])
    if not log:
        return
    total = sum(n for _, _, n in log)
    terminalreporter.write_line("routing flips (certified near-ties): %d over %d cases" %
                                (total, len(log)))
    for case, T, n in log:
        if n:
            terminalreporter.write_line("  %s: %d of %d tokens" % (case, n, T))
