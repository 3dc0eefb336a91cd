import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _keep_freed_memory_mapped():
    """The oracle checks of the full-size layers widen one expert's weights at a time to float64
    (hundreds of MB). glibc serves such blocks with fresh mmap pages and returns them on free, so
    every expert pays the page faults again, several times the cost of its arithmetic. Serving them
    from the heap and never trimming it keeps the pages (the peak stays what one expert needs)."""
    try:
        import ctypes
        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-3, 1 << 30)          # M_MMAP_THRESHOLD: blocks below 1 GiB come from the heap
        libc.mallopt(-1, (1 << 62) - 1)    # M_TRIM_THRESHOLD: never hand the heap top back
    except (OSError, AttributeError):     # pragma: no cover - not glibc
        pass


_keep_freed_memory_mapped()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size cases (minutes)")


def _ensure_built():
    """Build the shared libraries in-tree if they are missing (CPU-side, e.g. a fresh checkout)."""
    from synth import LIB_PATH as syn_lib
    if not os.path.exists(syn_lib):
        from synth import build as b
        b.build()
    lib = os.path.join(ROOT, "sparse_moe_layer_router_amd", "libmoe.so")
    if not os.path.exists(lib):
        # load the build script by path: importing the package itself requires the library
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_moe_build", os.path.join(ROOT, "sparse_moe_layer_router_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


_ensure_built()
