"""softmax_sink_amd -- sink attention for MI355X (gfx950).

The compute path is ``libsinkattn.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/sink_attn.h``). ``softmax_sink_amd.binding`` is the
thin ctypes layer over it; importing this package loads nothing, so the
seeded input generators in ``softmax_sink_amd.workloads`` stay usable on
machines without the library.
"""
import importlib

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
