import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _keep_freed_memory_in_heap():
    """Large numpy temporaries in the oracle otherwise page-fault afresh on every call."""
    import ctypes
    try:
        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-3, 32 << 20)  # M_MMAP_THRESHOLD: blocks below 32 MiB come from the heap
        libc.mallopt(-1, 1 << 30)   # M_TRIM_THRESHOLD: keep up to 1 GiB of freed heap
        libc.mallopt(-2, 64 << 20)  # M_TOP_PAD
    except (OSError, AttributeError):
        pass


_keep_freed_memory_in_heap()
