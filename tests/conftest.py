import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-only oracle test")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Error statistics of every GPU-vs-oracle comparison of this run (per-tensor relative
    error against its bound, per-element statistics), so that they stay in the log."""
    helpers = sys.modules.get("tests.gpu_helpers")
    stats = getattr(helpers, "PARITY_STATS", None)
    if not stats:
        return
    tr = terminalreporter
    tr.section("parity error statistics (GPU vs oracle)")
    tr.write_line(f"{'comparison':<44} {'dtype':<5} {'n':>9} {'err':>9} {'bound':>7} {'margin':>7} "
                  f"{'max_abs':>9} {'mean_abs':>9} {'p99/max':>9} {'>1ulp':>7}")
    for s in stats:
        margin = s["bound"] / s["err"] if s["err"] > 0 else float("inf")
        tr.write_line(f"{s['what'][:44]:<44} {s['dtype']:<5} {s['n']:>9} {s['err']:>9.2e} {s['bound']:>7.0e} "
                      f"{margin:>7.1f} {s['max_abs']:>9.2e} {s['mean_abs']:>9.2e} {s['p99_rel']:>9.2e} "
                      f"{s['gt_1ulp']:>7.4f}")
    worst = max(stats, key=lambda s: s["err"] / s["bound"])
    tr.write_line(f"{len(stats)} comparisons; smallest margin {worst['bound'] / max(worst['err'], 1e-300):.1f}x "
                  f"({worst['what']})")
