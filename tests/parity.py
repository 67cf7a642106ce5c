"""Shared parity machinery for the GPU tests: build inputs, run the HIP path
through the C ABI, and compare with the oracle at the stated tolerances.

Acceptance (the bar every GPU parity test applies):
* pages: byte-equal, except index fields whose oracle coordinate was within
  1e-6 of a codebook boundary, and those mismatches are fewer than 1e-4 of
  all written indices; norm bytes have no exemption;
* decode: max |gpu - oracle| <= 2e-3 and ||gpu - oracle||_2 / ||oracle||_2
  <= 1e-3 over the whole output, fp32 accumulation.
"""

from __future__ import annotations

import numpy as np

import oracle

DECODE_MAX_ABS = 2e-3
DECODE_REL_L2 = 1e-3
NEAR_FRACTION = 1e-4


def compare_pages(gpu_pages: np.ndarray, ref_pages: np.ndarray, near: np.ndarray, bits: int,
                  written_rows: int, d: int = 128, check_fraction: bool = True):
    """Assert the page bytes match the oracle's; returns (mismatched indices, total).

    ``check_fraction=False`` drops the 1e-4 bound on the number of
    near-boundary mismatches (for hand-made rows that sit on boundaries by
    construction); a mismatch away from a boundary always fails.
    """
    assert gpu_pages.shape == ref_pages.shape
    ib = oracle.index_bytes(d, bits)
    # norm bytes: exact
    gn = gpu_pages[..., ib:]
    rn = ref_pages[..., ib:]
    bad_norm = np.argwhere(np.any(gn != rn, axis=-1))
    assert len(bad_norm) == 0, f"norm bytes differ at {bad_norm[:5].tolist()}"
    if np.array_equal(gpu_pages, ref_pages):
        return 0, written_rows * d
    gi = oracle.unpack_indices(gpu_pages[..., :ib], bits, d)
    ri = oracle.unpack_indices(ref_pages[..., :ib], bits, d)
    diff = gi != ri
    # repacking the GPU's indices must give its bytes (no stray bits)
    assert np.array_equal(oracle.pack_indices(gi, bits), gpu_pages[..., :ib]), "stray bits in index bytes"
    assert not np.any(diff & ~near), f"index mismatch away from a boundary at {np.argwhere(diff & ~near)[:5].tolist()}"
    n_bad = int(diff.sum())
    total = written_rows * d
    if check_fraction:
        assert n_bad < NEAR_FRACTION * total, f"{n_bad} near-boundary mismatches of {total}"
    return n_bad, total


def compare_decode(out: np.ndarray, ref: np.ndarray, what: str = ""):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    diff = out - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff))
    worst = np.unravel_index(int(np.argmax(np.abs(diff))), diff.shape) if diff.size else None
    assert max_abs <= DECODE_MAX_ABS, f"{what}: max|d|={max_abs:.3e} at {worst}"
    assert rel <= DECODE_REL_L2, f"{what}: relL2={rel:.3e}"
    return max_abs, rel
