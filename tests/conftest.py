import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def pkv():
    """The product binding; builds libpkv.so first only when nothing is built."""
    lib_path = os.path.join(ROOT, "paged_kv_cache_346_amd", "libpkv.so")
    if not os.path.exists(lib_path):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_pkv_build", os.path.join(ROOT, "paged_kv_cache_346_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(verbose=False)
    import paged_kv_cache_346_amd
    host = os.environ.get("PKV_TEST_HOST_LIB")
    if host:
        # a host-only build of the block manager, scheduler, step packer and
        # planner (tests/test_host_sanitizers.py runs the host parity tests on
        # one built with AddressSanitizer and UndefinedBehaviorSanitizer): the
        # binding's host calls go to it
        import ctypes
        handle = ctypes.CDLL(host)
        for name, (res, args) in paged_kv_cache_346_amd.SIGNATURES.items():
            if hasattr(handle, name):
                fn = getattr(handle, name)
                fn.restype, fn.argtypes = res, args
        paged_kv_cache_346_amd.lib = handle
    return paged_kv_cache_346_amd
