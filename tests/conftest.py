import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU oracle check")


@pytest.fixture(autouse=True)
def _label_parity_stats(request):
    """Label the parity statistics a test records with the test's name."""
    mod = sys.modules.get("tests.parity_util")
    if mod is not None:
        mod.CURRENT_TEST = request.node.name
    yield


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Raw parity statistics of every GPU-vs-oracle comparison that ran: max |err| / RMS and the
    elements beyond 2e-3 RMS, split by what explains them (cast flip / accumulation bound)."""
    parity_util = sys.modules.get("tests.parity_util")
    if parity_util is None or not parity_util.STATS:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity statistics (raw error vs the 2e-3 RMS bar)")
    tr.write_line(f"{'case':34s} {'tensor':12s} {'max|err|/rms':>12s} {'n':>10s} {'>2e-3rms':>9s} "
                  f"{'flip':>7s} {'accum':>7s} {'norm unexpl':>11s}")
    for st in parity_util.STATS:
        tr.write_line(f"{st['case'][:34]:34s} {st['name'][:12]:12s} {st['max_err_over_rms']:12.3e} {st['n']:10d} "
                      f"{st['n_beyond_rel_rms']:9d} {st['n_flip_explained']:7d} {st['n_accumulation_explained']:7d} "
                      f"{st['norm_rel_unexplained']:11.2e}")
