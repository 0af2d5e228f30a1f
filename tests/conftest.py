import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The parity margins of the GPU tests (recorded by gpu_util.compare): max-abs and
    mean-abs error of O, max-abs error of LSE and relative L2 of O, per case, against
    the fp64 oracle."""
    mod = sys.modules.get("gpu_util")
    rows = getattr(mod, "MARGINS", None) if mod else None
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", f"parity margins ({len(rows)} comparisons against the fp64 oracle)")
    worst = {}
    for (what, dtype, mx, mean, lse, rel, n) in rows:
        tr.write_line(f"{what[:48]:48s} {dtype:4s} rows {n:6d} max-abs {mx:.2e} "
                      f"mean-abs {mean:.2e} lse {lse:.2e} rel-l2 {rel:.2e}")
        w = worst.setdefault(dtype, [0.0, 0.0, 0.0])
        worst[dtype] = [max(w[0], mx), max(w[1], mean), max(w[2], lse)]
    for dtype, (mx, mean, lse) in sorted(worst.items()):
        tr.write_line(f"worst {dtype}: max-abs {mx:.2e} mean-abs {mean:.2e} lse {lse:.2e}")
