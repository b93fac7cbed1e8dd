import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def golden():
    return load_golden


def pytest_sessionstart(session):
    """Build libpagedkv.so in-tree if it is missing (CPU cross-compile; the
    GPU runs always use a library built beforehand)."""
    lib = os.path.join(ROOT, "paged_kv_cache_136_amd", "libpagedkv.so")
    if not os.path.exists(lib):
        import runpy
        runpy.run_path(os.path.join(ROOT, "paged_kv_cache_136_amd", "build.py"))["build"]()


def pytest_terminal_summary(terminalreporter):
    """Print the figures GPU tests recorded (max abs errors of the full-size
    parity cases), so a run's log carries them even when every test passes."""
    mod = sys.modules.get("tests.gpu_util")
    rows = getattr(mod, "REPORT", [])
    if rows:
        terminalreporter.section("parity figures")
        for name, value in rows:
            terminalreporter.write_line(f"{name}: {value:.3e}")
