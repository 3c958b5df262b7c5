"""Batched generated-topology construction for MI355X (gfx950).

The compute path is the HIP library ``libtopo.so`` behind the C ABI in
``include/topo.h``; ``binding`` is its thin ctypes binding. Importing this
package does not load the library; the first binding call does, and fails
loudly when it has not been built (``python -m topology_construction_amd.build``).
"""
import importlib

from . import synth  # noqa: F401  (pure-numpy input generator)

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name == "binding":
        return importlib.import_module(".binding", __name__)
    raise AttributeError(name)
