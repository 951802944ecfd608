import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library through its C ABI")


def pytest_runtest_protocol(item, nextitem):
    # Name a GPU case before it runs, on the terminal (this hook runs outside
    # the output capture), so that a run that ends abruptly still says which
    # test was on the GPU.
    if item.get_closest_marker("gpu") is not None:
        tr = item.config.pluginmanager.get_plugin("terminalreporter")
        if tr is not None:
            tr.write_line(f"[gpu start] {item.nodeid}")
            tr._tw.flush()
    return None


def pytest_terminal_summary(terminalreporter):
    # Measured values that tests recorded with record_property("measured", ...)
    # (the timing gates), passed or failed, so that a regression shows as a
    # number in any run, -q included.
    lines = []
    for key in ("passed", "failed"):
        for rep in terminalreporter.stats.get(key, []):
            for name, value in getattr(rep, "user_properties", []):
                if name == "measured" and rep.when == "call":
                    lines.append(f"[measured] {rep.nodeid} ({key}): {json.dumps(value)}")
    if lines:
        terminalreporter.section("measured values")
        for line in lines:
            terminalreporter.write_line(line)
