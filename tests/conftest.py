import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _ensure_built():
    # Build only what is missing; a stale library is rebuilt by build().
    lib = os.path.join(ROOT, "w8a8_quantized_linear_quant_amd", "libw8a8.so")
    if not os.path.exists(lib):
        # by file path: importing the package would load the missing library
        import importlib.util

        spec = importlib.util.spec_from_file_location(
            "_w8a8_build", os.path.join(ROOT, "w8a8_quantized_linear_quant_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build_library()
    olib = os.path.join(ROOT, "oracle", "libw8a8_oracle.so")
    if not os.path.exists(olib):
        from oracle.build import build_oracle
        build_oracle()


_ensure_built()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
