import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU and the built libpa.so")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stderr (unbuffered) before it touches the GPU."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield


def pytest_terminal_summary(terminalreporter):
    """Worst |gpu - oracle| / (atol + rtol |oracle|) per checked label."""
    helpers = sys.modules.get("gpu_helpers")
    worst = getattr(helpers, "WORST_RATIO", None)
    if not worst:
        return
    terminalreporter.write_line("worst err/bound per checked label (1.0 = at tolerance):")
    for what, r in sorted(worst.items(), key=lambda kv: -kv[1]):
        terminalreporter.write_line(f"  {r:7.4f}  {what}")
