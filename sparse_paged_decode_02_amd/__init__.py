"""sda: DSA sparse decode attention over a paged KV cache, for MI355X (gfx950).

The compute path is libsda.so (HIP kernels behind a C ABI, include/sda.h);
this package is its thin ctypes binding.  Seeded synthetic workloads live in
``inputs``.
"""
from .binding import (  # noqa: F401
    SdaError,
    sda_decode,
    sda_splits,
    sda_workspace_bytes,
    status_string,
)
