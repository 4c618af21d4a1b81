"""MI355X (gfx950) causal prefill attention behind a C ABI.

The compute path is the hand-written HIP library ``libattn_prefill.so``
built from ``csrc/``; ``binding`` marshals arguments to its C entry points
with ctypes.  ``workloads`` draws seeded synthetic inputs and ``measure``
counts algorithmic work.  There is no CPU fallback: if the library is
missing, calling it raises.
"""
import importlib

__all__ = ["binding", "workloads", "measure"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
