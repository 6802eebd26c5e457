"""Partitioned attention over a static ring-buffer KV cache, for MI355X (gfx950).

The compute path is the HIP library ``libpattn.so`` (built from ``csrc/``)
behind a C ABI declared in ``include/pattn.h``. ``lib`` is its thin ctypes
binding; it raises if the library is missing and never falls back to a CPU
implementation. ``configs`` and ``synth`` (shapes and seeded inputs) need no
GPU and are importable anywhere.
"""

__all__ = ["configs", "synth", "lib"]


def __getattr__(name):
    if name == "lib":
        from . import _lib
        return _lib
    raise AttributeError(name)
