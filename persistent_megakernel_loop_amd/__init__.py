"""Persistent-megakernel batch-1 decode for AMD MI355X (gfx950).

The compute path is the HIP library ``libmk.so`` (C ABI in ``include/mk.h``);
``binding`` is a thin ctypes layer over it.  ``workload`` draws the seeded
synthetic inputs.
"""
from .binding import (  # noqa: F401
    MkError,
    Decoder,
    embed_sum,
    lib,
    library_path,
)
