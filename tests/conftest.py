import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the error figures the GPU parity tests recorded (raw and net y
    errors per layer, gradient errors per tensor), one line each."""
    harness = sys.modules.get("gpu_harness")
    rows = getattr(harness, "RESULTS", None)
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity figures (max|d|/rms for y: raw, and net of the output's own rounding; "
                      "|d|/|ref| for gradients)")
    def fmt(v):
        return ("%.4g" % v) if isinstance(v, float) else str(v)

    for last in (False, True):  # the full-size workloads close the output
        for kind, case, full, fig in rows:
            if full == last:
                tr.write_line("%-5s %-34s %s" % (kind, case, "  ".join("%s=%s" % (k, fmt(v)) for k, v in fig.items())))
