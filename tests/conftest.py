import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library through its C ABI")


def pytest_runtest_setup(item):
    # name a GPU case before it runs, so a run that ends abruptly still says
    # which test was on the GPU
    if item.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"[gpu start] {item.nodeid}\n")
        sys.__stderr__.flush()
