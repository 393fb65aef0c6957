"""Paged-KV decode attention for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libpa.so`` (hand-written HIP kernels,
declared in ``include/pa.h``).  This package holds its thin ctypes binding,
the host-side block pool and the seeded workload generators.  The binding is
loaded lazily so that the host-only modules import without the library.
"""

__all__ = [
    "pa_reshape_and_cache",
    "pa_copy_blocks",
    "pa_decode",
    "pa_decode_workspace_size",
    "pa_status_string",
    "PaError",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
