"""cross_layer_kv_amd -- FusedKV reconstruction-layer attention for MI355X (gfx950).

The compute lives in ``libfusedkv.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/fusedkv.h``).  ``binding`` is a thin ctypes layer
with the same entry-point names; ``inputs`` makes seeded synthetic inputs.
Importing the package does not load the library; the first call into
``binding`` does, and raises if the library has not been built.
"""
__all__ = ["binding", "inputs", "build"]


def __getattr__(name):
    if name in ("binding", "inputs", "build"):
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
