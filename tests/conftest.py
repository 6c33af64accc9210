import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Worst element-wise and norm-wise errors of every GPU-vs-oracle check that ran, so that the
    end of the run's output carries them."""
    harness = sys.modules.get("tests.harness")
    results = getattr(harness, "RESULTS", None)
    if not results:
        return
    tr = terminalreporter
    tr.write_sep("-", "GPU vs oracle: worst errors per check")
    tr.write_line(f"{'check':<58} {'rows':>7} {'max abs':>10} {'norm-wise':>10}")
    for what in sorted(results):
        a, n, rows = results[what]
        tr.write_line(f"{what[:58]:<58} {rows:>7} {a:>10.3e} {n:>10.3e}")
    worst_a = max(v[0] for v in results.values())
    worst_n = max(v[1] for v in results.values())
    tr.write_line(f"{len(results)} checks; worst max abs {worst_a:.3e}, worst norm-wise {worst_n:.3e}")
