"""GPU parity of the dense readback (tq_decompress_kv) against the oracle.

The readback reconstructs stored rows as n * s * (H c[idx]) / sqrt(d).  Each
case reads pages that the oracle wrote (or seeded random page bytes, which no
writer produced) and compares every output element with
``oracle.decompress_kv`` of the same page bytes, in float64:

* fp32 out: |gpu - oracle| <= 4e-6 * n + 2^-24 |oracle|, with n the row's
  stored norm.  The inverse transform runs in fp32: seven butterfly stages
  over centroids of magnitude <= 0.3 round to at most about
  7 * 128 * 0.3 * 2^-24 = 1.6e-5 before the factor n / sqrt(128), i.e.
  1.4e-6 * n;
* fp16 / bf16 out: the same plus one unit in the last place of the output
  format (2^-10 / 2^-7 relative; the GPU rounds its fp32 value once) and
  fp16's subnormal step 2^-24.

Negative slots must give zero rows; out-of-range slots zero rows and a count.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import api, workloads
from paged_decode_attention_tq_amd._lib import TQError

pytestmark = pytest.mark.gpu

_ULP = {torch.float32: 2.0 ** -24, torch.float16: 2.0 ** -10, torch.bfloat16: 2.0 ** -7}


@pytest.fixture(scope="module")
def ctx():
    return api.Context(128, 42)


def _norms(pages, slots):
    """Stored norm of every (token, head) read through the slots (0 for a negative slot)."""
    NB, BS, Hkv, RB = pages.shape
    s = np.where(slots >= 0, slots, 0)
    n = np.ascontiguousarray(pages[s // BS, s % BS][..., RB - 4:]).view("<f4")[..., 0].astype(np.float64)
    return np.where((slots >= 0)[:, None], n, 0.0)


def _check(got, ref, norms, dtype, what):
    g = got.float().cpu().numpy().astype(np.float64)
    tol = 4e-6 * norms[..., None] + _ULP[dtype] * np.abs(ref)
    if dtype == torch.float16:
        tol = tol + 2.0 ** -24
    d = np.abs(g - ref)
    bad = d > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond tolerance, worst "
                           f"{float((d - tol).max()):.3e} at {np.unravel_index(np.argmax(d - tol), d.shape)}")
    print(f"  {what}: max|d| {d.max():.3e}  max|d|/n {float((d / np.maximum(norms[..., None], 1e-30)).max()):.3e}",
          flush=True)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_oracle_pages_all_bits_and_dtypes(ctx, bits, dtype):
    # a ragged workload with dropped slots: written by the oracle writer, read
    # back through the same slots (row count not a multiple of 64)
    w = workloads.make_workload(f"rb{bits}", k_bits=bits, num_q_heads=6, num_kv_heads=3,
                                seq_lens=[45, 1, 130, 17], seed=50 + bits, drop_frac=0.1, lognormal_sigma=0.5)
    print(f"[decompress] bits={bits} dtype={dtype} N={w.num_tokens} Hkv=3", flush=True)
    codec = oracle.OracleCodec(128, 42)
    pages, _ = codec.write_kv(w.rows("k"), w.zero_pages(bits), w.slots, bits)
    ref = codec.decompress_kv(pages, w.slots, bits)
    got = api.decompress_kv(ctx, torch.from_numpy(pages).cuda(), torch.from_numpy(w.slots).cuda(), bits,
                            out_dtype=dtype)
    torch.cuda.synchronize()
    assert (w.slots < 0).any()
    assert not got[torch.from_numpy(w.slots < 0)].any()  # dropped tokens: zero rows
    _check(got, ref, _norms(pages, w.slots), dtype, f"K{bits} {dtype}")


def test_random_page_bytes_any_slot_order(ctx):
    # every index pattern is a valid row: seeded random bytes, slots in random
    # order with repeats and negatives
    bits, NB, BS, Hkv = 5, 40, 16, 4
    pages = workloads.random_pages(NB, BS, Hkv, 128, bits, seed=3)
    rng = np.random.default_rng(4)
    slots = rng.integers(-3, NB * BS, size=1001).astype(np.int64)
    print(f"[decompress] random bytes K{bits} N={len(slots)}", flush=True)
    ref = oracle.decompress_kv(pages, slots, bits, oracle.rht_signs(42, 128), oracle.OracleCodec(128, 42).centroids32(bits))
    got = api.decompress_kv(ctx, torch.from_numpy(pages).cuda(), torch.from_numpy(slots).cuda(), bits)
    torch.cuda.synchronize()
    _check(got, ref, _norms(pages, slots), torch.float32, "random bytes")


def test_gpu_written_pages_read_back(ctx):
    # the whole path: the GPU writer encodes, the readback reconstructs; rows
    # whose bytes equal the oracle's (all but near-boundary exemptions) must
    # read back as the oracle reconstructs them
    bits = 3
    w = workloads.make_workload("rbw", k_bits=bits, num_q_heads=8, num_kv_heads=2, seq_lens=[300, 77],
                                seed=61, outlier_frac=0.02)
    print(f"[decompress] gpu-written K{bits} N={w.num_tokens}", flush=True)
    codec = oracle.OracleCodec(128, 42)
    raw = w.rows("k")
    ref_pages, _ = codec.write_kv(raw, w.zero_pages(bits), w.slots, bits)
    pg = torch.zeros(w.page_shape(bits), dtype=torch.uint8, device="cuda")
    slots = torch.from_numpy(w.slots).cuda()
    api.write_kv(ctx, torch.from_numpy(raw).cuda(), pg, slots, bits)
    got = api.decompress_kv(ctx, pg, slots, bits)
    torch.cuda.synchronize()
    gp = pg.cpu().numpy()
    s = w.slots
    same = np.all(gp[s // 16, s % 16] == ref_pages[s // 16, s % 16], axis=-1)  # [N, Hkv]
    assert same.mean() > 0.99
    ref = codec.decompress_kv(ref_pages, s, bits)
    g = got.cpu().numpy().astype(np.float64)
    n = _norms(ref_pages, s)
    d = np.abs(g - ref)[same]
    assert (d <= 4e-6 * n[same][:, None] + 2.0 ** -24 * np.abs(ref[same])).all(), float(d.max())


def test_out_of_range_slots_and_empty(ctx):
    bits, NB, BS, Hkv = 4, 3, 16, 2
    pages = torch.from_numpy(workloads.random_pages(NB, BS, Hkv, 128, bits, seed=5)).cuda()
    slots = torch.tensor([0, 48, -1, 47, 1000, 5], dtype=torch.int64, device="cuda")
    print("[decompress] out-of-range slots", flush=True)
    with pytest.raises(TQError):
        api.decompress_kv(ctx, pages, slots, bits)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((6, Hkv, 128), float("nan"), device="cuda")
    api.decompress_kv(ctx, pages, slots, bits, out=out, err_count=err, check_slots=False)
    torch.cuda.synchronize()
    assert int(err.item()) == 2
    assert not out[1].any() and not out[2].any() and not out[4].any()
    assert torch.isfinite(out).all() and out[0].abs().sum() > 0
    e = api.decompress_kv(ctx, pages, torch.zeros(0, dtype=torch.int64, device="cuda"), bits)
    assert e.shape == (0, Hkv, 128)


@pytest.mark.parametrize("name,bits,dtype", [("long_context", 4, torch.float16), ("ragged_write", 3, torch.bfloat16)])
def test_full_size_sampled(ctx, name, bits, dtype):
    # the full page pool of the configuration (random page bytes), every token
    # read back in one call in the benchmark's launch shape; 4096 sampled
    # tokens (all heads) compared with the oracle
    w = workloads.preset(name)
    print(f"[decompress] full size {name} K{bits} N={w.num_tokens} Hkv={w.num_kv_heads} {dtype}", flush=True)
    pages = workloads.random_pages(w.num_blocks, w.block_size, w.num_kv_heads, 128, bits, seed=7)
    out = api.decompress_kv(ctx, torch.from_numpy(pages).cuda(), torch.from_numpy(w.slots).cuda(), bits,
                            out_dtype=dtype)
    torch.cuda.synchronize()
    pick = np.sort(np.random.default_rng(8).choice(w.num_tokens, size=4096, replace=False))
    pick[-1] = w.num_tokens - 1  # the last row of the grid
    s = w.slots[pick]
    ref = oracle.OracleCodec(128, 42).decompress_kv(pages, s, bits)
    _check(out[torch.from_numpy(pick).cuda()], ref, _norms(pages, s), dtype, f"{name} sampled")
