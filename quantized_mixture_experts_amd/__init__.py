"""MI355X-native routed, weight-quantized MoE expert FFN.

The compute lives in a HIP/C++ shared library (``libqmoe.so``, gfx950) behind a
C ABI declared in ``include/qmoe.h``; ``binding`` marshals torch tensors into it.
``inputs`` draws the seeded synthetic workloads. Importing this package does not
load the library; the first call into ``binding`` does, and fails loudly if the
library is missing.
"""
import importlib

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
