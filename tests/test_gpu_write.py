"""GPU parity of the row writer (tq_write_kv) against the oracle, bit-exact up
to the near-boundary exemption."""

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import api, workloads
from tests.parity import compare_pages

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    return api.Context(128, 42)


@pytest.fixture(scope="module")
def codec():
    return oracle.OracleCodec(128, 42)


def _gpu_write(ctx, raw, pages, slots, bits, err=None, check=True):
    raw_t = raw if isinstance(raw, torch.Tensor) else torch.from_numpy(raw)
    pages_t = torch.from_numpy(pages).cuda()
    slots_t = torch.from_numpy(slots).cuda()
    api.write_kv(ctx, raw_t.cuda(), pages_t, slots_t, bits, err_count=err, check_slots=check)
    torch.cuda.synchronize()
    return pages_t.cpu().numpy()


def _check(ctx, codec, raw_np, pages0, slots, bits, raw_gpu=None, check_fraction=True):
    ref, near = codec.write_kv(raw_np, pages0, slots, bits)
    got = _gpu_write(ctx, raw_np if raw_gpu is None else raw_gpu, pages0, slots, bits)
    written = int((slots >= 0).sum()) * raw_np.shape[1]
    return compare_pages(got, ref, near, bits, written, check_fraction=check_fraction)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_write_matches_oracle(ctx, codec, bits, dtype):
    w = workloads.make_workload("w", k_bits=bits, num_q_heads=6, num_kv_heads=3, seq_lens=[70, 1, 33, 16],
                                dtype=dtype, seed=11 + bits, lognormal_sigma=0.5, drop_frac=0.1, extra_blocks=3)
    raw = w.rows("k")
    pages0 = np.random.default_rng(bits).integers(0, 256, size=w.page_shape(bits), dtype=np.uint8)
    print(f"[write] bits={bits} dtype={np.dtype(dtype).name} rows={raw.shape}", flush=True)
    n_bad, total = _check(ctx, codec, raw, pages0, w.slots, bits)
    print(f"  near-boundary mismatches {n_bad}/{total}")


@pytest.mark.parametrize("bits", [3, 4])
def test_write_bf16_input(ctx, codec, bits):
    t = torch.randn(40, 2, 128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    raw32 = t.float().numpy()  # bf16 values are exact in fp32
    slots = np.arange(40, dtype=np.int64)[::-1].copy()
    pages0 = np.zeros((3, 16, 2, oracle.row_bytes(128, bits)), np.uint8)
    _check(ctx, codec, raw32, pages0, slots, bits, raw_gpu=t)


def _special_rows(dtype):
    # zero row; a row whose norm is an exact fp32 tie (sqrt(1 + 2^-23 + 2^-48) =
    # 1 + 2^-24, the midpoint of 1 and 1 + 2^-23), which takes the exact
    # re-summation path; a one-hot row; constant rows; extreme magnitudes.
    d = 128
    rng = np.random.default_rng(1)
    x = np.zeros((8, 1, d), np.float64)
    x[1, 0, [0, 1, 2, 3]] = [1.0, 2.0**-12, 2.0**-12, 2.0**-24]
    x[2, 0, 77] = -3.0
    x[3, 0] = 1.0
    x[4, 0, ::2] = 0.5
    x[5, 0] = rng.standard_normal(d)
    if dtype == np.float32:
        x[6, 0] = rng.standard_normal(d) * 1e-20
        x[7, 0] = rng.standard_normal(d) * 1e18
    else:
        x[6, 0] = rng.integers(1, 30, d) * 2.0**-24  # fp16 subnormals
        x[7, 0] = rng.standard_normal(d) * 1e4
    return x.astype(dtype)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_write_special_rows(ctx, codec, bits, dtype):
    x = _special_rows(dtype)
    pages0 = np.zeros((1, 8, 1, oracle.row_bytes(128, bits)), np.uint8)
    # structured rows put rotated coordinates on or next to boundaries by
    # construction, so only the placement of mismatches is checked here
    n_bad, _ = _check(ctx, codec, x, pages0, np.arange(8, dtype=np.int64), bits, check_fraction=False)
    print(f"[special rows] bits={bits} {np.dtype(dtype).name}: near-boundary mismatches {n_bad}")
    _, n32, _, _ = codec.encode(x[1], bits)
    assert n32[0] == np.float32(1.0)  # the tie rounds to even


def test_out_of_range_slots_are_counted_and_never_written(ctx, codec):
    bits, NB, BS, H = 4, 3, 16, 2
    RB = oracle.row_bytes(128, bits)
    guard = torch.full((NB + 1, BS, H, RB), 0xAB, dtype=torch.uint8, device="cuda")
    pages = guard[:NB]
    raw = torch.randn(6, H, 128, device="cuda", dtype=torch.float16)
    slots = torch.tensor([0, NB * BS, 5, -3, NB * BS + 7, 47], dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.write_kv(ctx, raw, pages, slots, bits, err_count=err, check_slots=False)
    torch.cuda.synchronize()
    assert int(err.item()) == 2
    g = guard.cpu().numpy()
    assert np.all(g[NB] == 0xAB), "guard page written"
    ref, near = codec.write_kv(raw.cpu().numpy(), np.full((NB, BS, H, RB), 0xAB, np.uint8),
                               np.array([0, -1, 5, -3, -1, 47]), bits)
    compare_pages(g[:NB], ref, near, bits, 3 * H)
    with pytest.raises(api.TQError):
        api.write_kv(ctx, raw, pages, slots, bits)


def test_tiny_preset_pages(ctx, codec):
    w = workloads.preset("tiny")
    for comp in ("k", "v"):
        _check(ctx, codec, w.rows(comp), w.zero_pages(4), w.slots, 4)


@pytest.mark.parametrize("kb,vb,dtype", [(4, 4, torch.float16), (4, 2, torch.float16), (3, 5, torch.float32),
                                         (2, 3, torch.bfloat16)])
def test_write_pair_equals_two_writes_and_oracle(ctx, codec, kb, vb, dtype):
    # one launch for K and V gives the bytes of two single-component writes,
    # which match the oracle; a bad slot is skipped by both and counted once
    w = workloads.make_workload("pair", k_bits=kb, v_bits=vb, num_q_heads=8, num_kv_heads=4,
                                seq_lens=[37, 16, 5], seed=31 + kb + vb, drop_frac=0.1, extra_blocks=2)
    print(f"[write pair] K{kb}V{vb} {dtype} rows={w.num_tokens}x{w.num_kv_heads}", flush=True)
    kraw = torch.from_numpy(w.rows("k")).to(dtype)
    vraw = torch.from_numpy(w.rows("v")).to(dtype)
    slots = w.slots.copy()
    NB, BS = w.page_shape(kb)[:2]
    slots[3] = NB * BS + 1  # out of range
    slots_t = torch.from_numpy(slots).cuda()
    k0 = np.random.default_rng(kb).integers(0, 256, size=w.page_shape(kb), dtype=np.uint8)
    v0 = np.random.default_rng(vb + 9).integers(0, 256, size=w.page_shape(vb), dtype=np.uint8)
    kp, vp = torch.from_numpy(k0).cuda(), torch.from_numpy(v0).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.write_kv_pair(ctx, kraw.cuda(), vraw.cuda(), kp, vp, slots_t, kb, vb, err_count=err, check_slots=False)
    kp1, vp1 = torch.from_numpy(k0).cuda(), torch.from_numpy(v0).cuda()
    api.write_kv(ctx, kraw.cuda(), kp1, slots_t, kb, check_slots=False)
    api.write_kv(ctx, vraw.cuda(), vp1, slots_t, vb, check_slots=False)
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    assert np.array_equal(kp.cpu().numpy(), kp1.cpu().numpy())
    assert np.array_equal(vp.cpu().numpy(), vp1.cpu().numpy())
    ok = slots.copy()
    ok[3] = -1
    written = int((ok >= 0).sum()) * w.num_kv_heads
    for raw, pages0, got, bits in ((kraw, k0, kp, kb), (vraw, v0, vp, vb)):
        ref, near = codec.write_kv(raw.float().numpy(), pages0, ok, bits)
        compare_pages(got.cpu().numpy(), ref, near, bits, written)
    with pytest.raises(api.TQError):
        api.write_kv_pair(ctx, kraw.cuda(), vraw.cuda(), kp, vp, slots_t, kb, vb)
