"""CPU oracle for the TurboQuant packed-page KV path.

TEST INFRASTRUCTURE ONLY.  Nothing here is part of the product path: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library (no
kernels, headers, tables or constant generators); the only thing both sides
consume is the seeded input data produced by
``paged_decode_attention_tq_amd.workloads``.

Everything is plain numpy / scipy in float64 (mpmath for the final digits of
the codebook), written from the documentation pages of the ``turboquant``
package:

* "vLLM Usage" -- sections "TQ Byte Layout" (row = bit-packed indices + fp32
  norm), "Slot Mapping" (flat slots, negative ignored, out-of-range raises)
  and "TQ Packed Page Contract" (RHT rotation with seed 42, Lloyd-Max
  centroids, ``write_tq4_kv`` / ``decode_tq4_paged``);
* "vLLM Reference Audit" -- "Feature Checklist" (Lloyd-Max codebooks with
  exact Beta tests, RHT transforms, 1..5-bit packing);
* "Architecture" -- "Cache Storage Objects" (page shape
  ``[num_blocks, block_size, num_kv_heads, row_bytes]``) and "Diagnostic vs
  Serving Paths" (the paged decode reconstructs rows inside the loop).

Where the pages only name a step, the reading taken is stated in the
function that implements it.  Pins for every function live in
``tests/test_oracle_*.py``; no function here is "parity unpinned" except the
choice of pseudo-random generator behind the rotation seed (the pages do not
print their generator; see ``rht.rht_signs``).
"""

from .codebook import beta_codebook, gaussian_lloyd_max, lloyd_max_iterate
from .rht import splitmix64, rht_signs, fwht, rht, irht
from .codec import (
    row_bytes,
    index_bytes,
    encode_rows,
    pack_indices,
    unpack_indices,
    rows_to_bytes,
    bytes_to_rows,
    dequantize_rows,
    write_kv,
    decompress_kv,
    OracleCodec,
)
from .attention import paged_decode, paged_decode_heads, paged_decode_hybrid, paged_prefill
from .qjl import (
    prod_row_bytes,
    encode_prod,
    prod_rows_to_bytes,
    prod_bytes_to_rows,
    prod_scores,
    write_prod,
    paged_prod_scores,
)

__all__ = [
    "beta_codebook",
    "gaussian_lloyd_max",
    "lloyd_max_iterate",
    "splitmix64",
    "rht_signs",
    "fwht",
    "rht",
    "irht",
    "row_bytes",
    "index_bytes",
    "encode_rows",
    "pack_indices",
    "unpack_indices",
    "rows_to_bytes",
    "bytes_to_rows",
    "dequantize_rows",
    "write_kv",
    "decompress_kv",
    "OracleCodec",
    "paged_decode",
    "paged_decode_heads",
    "paged_decode_hybrid",
    "paged_prefill",
    "prod_row_bytes",
    "encode_prod",
    "prod_rows_to_bytes",
    "prod_bytes_to_rows",
    "prod_scores",
    "write_prod",
    "paged_prod_scores",
]
