"""Routed Mixture-of-Experts FFN forward for one MI355X (gfx950).

The compute path is libmoe.so: hand-written HIP kernels behind a C ABI declared in
include/moe.h. `binding` marshals torch tensors into that ABI; `inputs` generates the
seeded synthetic workloads. The binding is imported lazily so that the input generator
can be used on machines without the built library.
"""
import importlib

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in ("binding", "inputs"):
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
