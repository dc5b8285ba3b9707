import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The largest fp8 logit error seen per (head_dim, heads), in units of
    2^-23 A, against the allowance the comparisons use."""
    mod = sys.modules.get("gpu_helpers")
    units = getattr(mod, "FP8_UNITS", None) if mod else None
    if not units:
        return
    terminalreporter.write_line("fp8 logit error, largest observed (units of 2^-23 A) / allowance:")
    for (d, h), u in sorted(units.items()):
        terminalreporter.write_line(f"  [fp8-units] D={d} H={h}: {u:.1f} / {max(d, 128) + h + 2}")
