"""ZHA tree-indexed sparse decode on MI355X (gfx950).

The compute path is the HIP library libzha.so (C ABI declared in include/zha.h);
`binding` marshals arguments to it.  `workloads` draws the seeded inputs.
The binding is imported lazily so that CPU-only tools can use `workloads`.
"""
import importlib

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
