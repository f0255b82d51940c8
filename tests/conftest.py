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
        # by file path: the package's __init__ refuses to run without the library
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_moe_build", os.path.join(ROOT, "quantized_moe_routed_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
