import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_sessionstart(session):
    import util
    util._reporter = session.config.pluginmanager.getplugin("terminalreporter")
    util._capman = session.config.pluginmanager.getplugin("capturemanager")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Names each GPU case on the terminal before it runs, so that a run
    that ends abruptly still says which case was running."""
    if request.node.get_closest_marker("gpu") is not None:
        import util
        util.progress(f"[gpu case] {request.node.nodeid}")
    yield
