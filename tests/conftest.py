import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


import pytest  # noqa: E402


@pytest.fixture
def canaries(monkeypatch):
    """Every device buffer a test allocates through gemm_chains_amd.device.empty_bytes /
    empty_f32 (outputs, workspaces, packed weights) gets canary bytes on both sides, checked
    after the test."""
    import torch
    if not torch.cuda.is_available():
        yield None
        return
    from gemm_chains_amd import device
    from tests.helpers import Canaries
    cz = Canaries()
    monkeypatch.setattr(device, "empty_bytes", cz.bytes)
    monkeypatch.setattr(device, "empty_f32", cz.f32)
    yield cz
    cz.check()


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the parity figures the tests recorded (end-to-end errors, teacher-forced worst
    cases, converter counts), also under -q."""
    try:
        from tests.helpers import FIGURES
    except Exception:
        return
    if not FIGURES:
        return
    terminalreporter.write_sep("-", "parity figures")
    for label in sorted(FIGURES):
        terminalreporter.write_line(f"{label}: {FIGURES[label]}")
