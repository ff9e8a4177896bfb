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
        from . import binding
        if name == "binding":
            return binding
        return getattr(binding, name)
    raise AttributeError(name)
