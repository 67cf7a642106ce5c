"""TurboQuant packed-page KV path for AMD Instinct MI355X (gfx950).

``api`` holds the Python entry points over the C ABI of ``libtq.so``
(include/tq.h); ``workloads`` holds the seeded synthetic inputs.
"""

from .api import (  # noqa: F401
    TQError,
    Context,
    codebook,
    decode_kernel,
    decode_workspace_bytes,
    paged_decode,
    rht_signs,
    row_bytes,
    write_kv,
    write_kv_pair,
)
