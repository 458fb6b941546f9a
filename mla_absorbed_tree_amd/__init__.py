"""MI355X (gfx950) tree-verify attention for absorbed-form MLA.

The compute lives in libmlaverify.so (hand-written HIP kernels behind a C-ABI,
declared in include/mla_verify.h). `binding` forwards the C entry points
through ctypes; `verify.MlaVerify` owns a plan and its workspace. Both load the
library on first use and fail loudly when it has not been built.
"""
import importlib

__all__ = ["binding", "verify"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
