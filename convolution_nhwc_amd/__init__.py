"""MI355X (gfx950) NHWC convolution: forward and backward-data over fp16/bf16.

The compute runs in the HIP library ``libcnhwc.so`` behind a C ABI
(``include/cnhwc.h``); ``convolution_nhwc_amd.api`` is its thin ctypes binding.
Importing this package loads nothing; the binding is loaded on first use and
raises if the library has not been built.
"""
import importlib

__all__ = ["api", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
