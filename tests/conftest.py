import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The worst row and elementwise errors of the bf16 parity checks, per
    test function (parameters folded), so a GPU log keeps the figures."""
    gu = sys.modules.get("gpu_util")
    if gu is None or not gu.RESULTS:
        return
    worst = {}
    for r in gu.RESULTS:
        key = r["test"].split("[")[0].split("::")[-1]
        w = worst.setdefault(key, dict(checks=0, elements=0, max_err=0.0, elem_err=0.0, elem_what=""))
        w["checks"] += 1
        w["elements"] += r["elements"]
        w["max_err"] = max(w["max_err"], r["max_err"])
        if r["elem_err"] >= w["elem_err"]:
            w["elem_err"], w["elem_what"] = r["elem_err"], r["what"]
    tr = terminalreporter
    tr.write_sep("-", "bf16 parity: worst row / elementwise error per test")
    for key, w in sorted(worst.items()):
        tr.write_line(f"{key}: {w['checks']} checks, {w['elements']} elements, row {w['max_err']:.4f}, "
                      f"elem {w['elem_err']:.4f} ({w['elem_what']})")
    path = os.environ.get("MUSE_PARITY_REPORT")
    if path:
        import json
        with open(path, "w") as f:
            json.dump(gu.RESULTS, f)
