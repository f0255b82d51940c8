import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C ABI on the GPU)")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_sessionstart(session):
    # the library is built in-tree; compile it once if nothing is built yet
    lib = os.path.join(ROOT, "quantized_moe_routed_amd", "libmoe.so")
    if not os.path.exists(lib):
        from quantized_moe_routed_amd import build as _b
        _b.build()
