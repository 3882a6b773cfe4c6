import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the parity metrics of every named comparison as JSON lines (one
    per comparison, then one line holding the five workloads), so they
    survive ``pytest -q``; also write them to gpurun_out/parity_metrics.json
    when that folder exists."""
    mod = sys.modules.get("tests.parity")
    if mod is None or not mod.RECORDED:
        return
    rec = mod.RECORDED
    tr = terminalreporter
    tr.write_sep("-", "parity metrics")
    for name, m in rec.items():
        tr.write_line("[parity-metrics] " + json.dumps({"name": name, **m}, default=float))
    five = {k: {kk: rec[k][kk] for kk in ("max_abs", "max_abs_representable", "rel_l2", "max_dlse",
                                         "bf16_floor_max", "unrepresentable", "rows")}
            for k in rec if k.startswith("workload:")}
    if five:
        tr.write_line("[parity-workloads] " + json.dumps(five, default=float))
    out = os.path.join(ROOT, "gpurun_out")
    if os.path.isdir(out):
        with open(os.path.join(out, "parity_metrics.json"), "w") as f:
            json.dump(rec, f, indent=1, default=float)
