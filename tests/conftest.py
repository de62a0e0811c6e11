import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Repeat the GPU tests' measured margins (err/rms per workload) at the end of the output."""
    mod = sys.modules.get("tests._gpu_common")
    lines = getattr(mod, "SUMMARY", None) if mod else None
    if lines:
        terminalreporter.write_line("GPU parity margins (max|y - y_oracle| / rms against the bar):")
        for line in lines:
            if "err/rms" in line or "nan y" in line:
                terminalreporter.write_line("  " + line)
