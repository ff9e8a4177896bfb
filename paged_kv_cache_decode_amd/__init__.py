"""Paged-KV-cache attention for AMD MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pa.h``); ``binding`` marshals torch tensors into that
ABI.  ``workloads`` holds the seeded synthetic input generators.

The binding is imported lazily so that the input generators can be used on
machines without the built library.
"""

from . import workloads  # noqa: F401

__all__ = ["workloads", "binding", "decode", "prefill", "write_kv"]


def __getattr__(name):
    if name in ("binding", "decode", "prefill", "write_kv"):
        import importlib
        mod = importlib.import_module(__name__ + ".binding")
        return mod if name == "binding" else getattr(mod, name)
    raise AttributeError(name)
