"""sda: DSA sparse decode attention over a paged KV cache, for MI355X (gfx950).

The compute path is libsda.so (HIP kernels behind a C ABI, include/sda.h);
this package is its thin ctypes binding.  ``sda_decode`` is the sparse decode
of the DSA layers, ``sda_select_regions`` the region selection upstream of it,
``sda_indexer_logits`` the region scores upstream of that,
and ``sda_swa_decode`` the gated sliding-window decode of the other layers over
the same cache.  Seeded synthetic workloads live in
``inputs``.
"""
from .binding import (  # noqa: F401
    SdaError,
    sda_decode,
    sda_decode_static,
    sda_device_compute_units,
    sda_indexer_logits,
    sda_select_regions,
    sda_splits,
    sda_swa_decode,
    sda_swa_plan,
    sda_workspace_bytes,
    status_string,
)
