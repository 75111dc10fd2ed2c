"""Shared pytest setup: repo root on sys.path and the ``gpu`` marker."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


def pytest_terminal_summary(terminalreporter):
    """Worst per-unit output error ratio of the GPU parity checks of this session."""
    harness = sys.modules.get("decode_harness")
    worst = getattr(harness, "WORST_UNIT", None) if harness else None
    if worst:
        terminalreporter.section("per-unit output error (max|out-ref| / max|ref| per (sequence, KV head))")
        for kv, (ratio, where) in sorted(worst.items()):
            terminalreporter.write_line(f"{kv}: worst {ratio:.3e} (bound {harness.UNIT_TOL:g}) in {where}")
