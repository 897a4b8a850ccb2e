"""pytest plugin (``-p tests.san_plugin``): binds the package's host-side pool
calls to the library named by ``PA_SAN_POOL_LIB``, a host-only build of
``pa_pool.cpp`` made with AddressSanitizer and UndefinedBehaviorSanitizer, so
that the pool's CPU tests run under both.  Loaded only by
tests/test_sanitizers.py, in a child process started with the ASan runtime
preloaded; the library has the pool's symbols and no device code.
"""
import ctypes
import os

import paged_kv_cache_06_amd as pa


def pytest_configure(config):
    lib = ctypes.CDLL(os.environ["PA_SAN_POOL_LIB"])
    bound = 0
    for name, (res, args) in pa._SIGNATURES.items():
        fn = getattr(lib, name, None)
        if fn is None:  # a device entry point: not in the host-only build
            continue
        fn.restype = res
        fn.argtypes = args
        bound += 1
    assert bound >= 15, f"only {bound} pool symbols in {os.environ['PA_SAN_POOL_LIB']}"
    pa._lib = lib
