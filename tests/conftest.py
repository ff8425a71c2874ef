import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The comparison statistics of every attention check of the run (max-abs
    error, max-rel error over |o| >= 0.1, RMS error), one line per check, and
    the worst of each per dtype."""
    mod = sys.modules.get("gpu_util")
    stats = getattr(mod, "STATS", None) if mod else None
    if not stats:
        return
    tr = terminalreporter
    tr.section("attention parity statistics (kernel vs fp64 oracle)")
    worst = {}
    for what, dtype, st in stats:
        rel = "-" if st["max_rel"] is None else f"{st['max_rel']:.3e}"
        tr.write_line(f"{dtype:5s} n={st['n']:>10d} max_abs={st['max_abs']:.3e} max_rel={rel} rms={st['rms']:.3e}  "
                      f"{what}")
        w = worst.setdefault(dtype, {"max_abs": 0.0, "max_rel": 0.0, "rms": 0.0, "checks": 0})
        w["checks"] += 1
        w["max_abs"] = max(w["max_abs"], st["max_abs"])
        w["rms"] = max(w["rms"], st["rms"])
        if st["max_rel"] is not None:
            w["max_rel"] = max(w["max_rel"], st["max_rel"])
    for dtype, w in worst.items():
        tr.write_line(f"worst {dtype}: {w['checks']} checks, max_abs {w['max_abs']:.3e}, max_rel (|o| >= 0.1) "
                      f"{w['max_rel']:.3e}, rms {w['rms']:.3e}")
