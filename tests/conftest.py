import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Parity margins of the GPU tests that ran (normwise error against its tolerance,
    and the element-wise error with a floor of 1 % of the row's largest value)."""
    helpers = sys.modules.get("gpu_helpers")
    rows = getattr(helpers, "MARGINS", None) if helpers else None
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity margins (normwise / tolerance, element-wise)")
    for r in rows:
        el = "" if r["elementwise"] is None else f"  elem {r['elementwise']:.2e}"
        nt = "" if r["n_tokens"] is None else f"  N={r['n_tokens']}"
        tr.write_line(f"{r['case']}: {r['normwise']:.2e} / {r['tol']:g}"
                      f" ({r['normwise'] / r['tol']:.0%}){el}{nt}")
