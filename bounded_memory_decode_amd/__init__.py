"""MI355X-native Rock Memory Anchors (RMA) layer step.

The compute lives in ``librma.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/rma.h``); ``bounded_memory_decode_amd.rma`` is the
thin ctypes binding.  ``synth`` holds the seeded synthetic inputs.
Submodules are imported on demand so that ``synth`` can be used without
loading the HIP library.
"""
__all__ = ["rma", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
