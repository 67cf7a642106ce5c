"""GPU parity of the paged decode (tq_paged_decode) against the oracle.

Each case runs the decode on pages written by the oracle (isolating the
decode) and on pages written by the GPU writer (the whole path), and checks
max-abs <= 2e-3 and rel-L2 <= 1e-3 against the oracle's output.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import api, workloads
from tests.parity import compare_decode, compare_pages

pytestmark = pytest.mark.gpu

_TORCH = {np.float16: torch.float16, np.float32: torch.float32}


@pytest.fixture(scope="module")
def ctx():
    return api.Context(128, 42)


def _oracle_pipeline(w, with_near=False):
    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    kraw, vraw = w.rows("k"), w.rows("v")
    kp, near_k = codec.write_kv(kraw, w.zero_pages(w.k_bits), w.slots, w.k_bits)
    vp, near_v = codec.write_kv(vraw, w.zero_pages(w.v_bits), w.slots, w.v_bits)
    if with_near:
        return codec, kraw, vraw, kp, vp, near_k, near_v
    return codec, kraw, vraw, kp, vp


def _decode(ctx, w, q, kp, vp, scale=None):
    out = api.paged_decode(
        ctx, q, kp, vp, torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(),
        w.k_bits, w.v_bits, max_seq_len=w.max_seq_len, scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _run(ctx, w, scale=None, q_dtype=None, gpu_write=True):
    print(f"[decode] {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"K{w.k_bits}V{w.v_bits} lens={w.seq_lens[:8].tolist()} scale={scale}", flush=True)
    codec, kraw, vraw, kp, vp, near_k, near_v = _oracle_pipeline(w, with_near=True)
    q = w.queries()
    ref = oracle.paged_decode(q, kp, vp, w.block_table, w.seq_lens, w.k_bits, w.v_bits, codec.signs,
                              codec.centroids32(w.k_bits), codec.centroids32(w.v_bits), scale)
    qt = torch.from_numpy(q).cuda()
    if q_dtype is not None:
        qt = qt.to(q_dtype)
        ref = oracle.paged_decode(qt.float().cpu().numpy(), kp, vp, w.block_table, w.seq_lens, w.k_bits,
                                  w.v_bits, codec.signs, codec.centroids32(w.k_bits),
                                  codec.centroids32(w.v_bits), scale)
    out = _decode(ctx, w, qt, torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda(), scale)
    r1 = compare_decode(out, ref, f"{w.name} oracle pages")
    r2 = None
    if gpu_write:
        kpg = torch.zeros(w.page_shape(w.k_bits), dtype=torch.uint8, device="cuda")
        vpg = torch.zeros(w.page_shape(w.v_bits), dtype=torch.uint8, device="cuda")
        slots = torch.from_numpy(w.slots).cuda()
        api.write_kv(ctx, torch.from_numpy(kraw).cuda(), kpg, slots, w.k_bits)
        api.write_kv(ctx, torch.from_numpy(vraw).cuda(), vpg, slots, w.v_bits)
        # the GPU-written pages are the oracle's, byte for byte (near-boundary exemption)
        written = int((w.slots >= 0).sum()) * w.num_kv_heads
        compare_pages(kpg.cpu().numpy(), kp, near_k, w.k_bits, written)
        compare_pages(vpg.cpu().numpy(), vp, near_v, w.v_bits, written)
        out2 = _decode(ctx, w, qt, kpg, vpg, scale)
        r2 = compare_decode(out2, ref, f"{w.name} gpu pages")
    print(f"  max|d| relL2 oracle-pages {r1}  gpu-pages {r2}", flush=True)
    return out, ref


@pytest.mark.parametrize("kb,vb", [(4, 4), (4, 2), (3, 3), (5, 5), (2, 5), (5, 3), (2, 2)])
def test_bits_combinations(ctx, kb, vb):
    w = workloads.make_workload(f"bits{kb}{vb}", k_bits=kb, v_bits=vb, num_q_heads=16, num_kv_heads=2,
                                seq_lens=[300, 17, 1, 64, 0, 129], seed=kb * 10 + vb, lognormal_sigma=0.5)
    _run(ctx, w)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 16, 64])
def test_group_sizes(ctx, G):
    w = workloads.make_workload(f"group{G}", num_q_heads=2 * G, num_kv_heads=2, seq_lens=[200, 45, 16],
                                seed=G, outlier_frac=0.02)
    _run(ctx, w)


@pytest.mark.parametrize("hkv,G,kb,vb", [(32, 1, 4, 4), (4, 40, 4, 2), (6, 24, 3, 5), (16, 1, 2, 3)])
def test_kv_head_slices(ctx, hkv, G, kb, vb):
    # more KV heads x query groups than one workgroup holds: each workgroup
    # stages per-token slices of its heads (including 4- and 8-byte misalignments)
    w = workloads.make_workload(f"slices{hkv}x{G}", k_bits=kb, v_bits=vb, num_q_heads=hkv * G, num_kv_heads=hkv,
                                seq_lens=[130, 47, 300], seed=hkv + G)
    _run(ctx, w)


def test_many_splits_and_ragged_tails(ctx):
    # long enough for many 16-page splits per sequence, with ragged last pages
    w = workloads.make_workload("splits", num_q_heads=8, num_kv_heads=1, seq_lens=[9000, 4097, 255, 16, 15],
                                seed=5, extra_blocks=5)
    _run(ctx, w)


def test_tiny_preset(ctx):
    _run(ctx, workloads.preset("tiny"))


@pytest.mark.parametrize("name,kw", [
    ("pages_geometry", dict(batch=3, seq_len=600)),
    ("mixed_bits", dict(batch=3, seq_len=700)),
    ("long_context", dict(batch=1, seq_len=5000)),
    ("ragged_write", dict(batch=6, len_range=(1, 3000))),
])
def test_presets_at_reduced_size(ctx, name, kw):
    _run(ctx, workloads.preset(name, **kw))


@pytest.mark.parametrize("q_dtype", [torch.float32, torch.bfloat16])
def test_query_dtypes(ctx, q_dtype):
    w = workloads.make_workload("qdt", num_q_heads=8, num_kv_heads=2, seq_lens=[100, 33], seed=9)
    _run(ctx, w, q_dtype=q_dtype, gpu_write=False)


def test_scale_override(ctx):
    w = workloads.make_workload("scale", num_q_heads=8, num_kv_heads=2, seq_lens=[100, 33], seed=10)
    _run(ctx, w, scale=0.3)


def test_zero_and_single_token_sequences(ctx):
    w = workloads.make_workload("edge", num_q_heads=4, num_kv_heads=2, seq_lens=[0, 1, 0, 2], seed=12)
    out, ref = _run(ctx, w)
    assert not out[0].any() and not out[2].any()


@pytest.mark.parametrize("B,hkv,G", [(3, 2, 8), (70, 1, 4), (5, 8, 8)])
def test_all_sequences_empty(ctx, B, hkv, G):
    # every length 0: the output is all zeros, written over whatever out held
    # (one-workgroup wave decode, a batch past its 64-sequence bound, staged)
    dev = torch.device("cuda")
    rb = 68
    kp = torch.zeros((2, 16, hkv, rb), dtype=torch.uint8, device=dev)
    vp = torch.zeros_like(kp)
    q = torch.randn((B, hkv * G, 128), dtype=torch.float16, device=dev)
    bt = torch.zeros((B, 1), dtype=torch.int32, device=dev)
    lens = torch.zeros(B, dtype=torch.int32, device=dev)
    out = torch.full((B, hkv * G, 128), float("nan"), dtype=torch.float32, device=dev)
    print(f"[empty] B={B} Hkv={hkv} G={G} kernel={api.decode_kernel(B, hkv * G, hkv, 0, 4, 4)}", flush=True)
    api.paged_decode(ctx, q, kp, vp, bt, lens, 4, 4, max_seq_len=0, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_large_and_small_norms(ctx):
    # values far from unit scale: weights must neither overflow nor lose precision
    for sigma, scale_raw, q_mul in ((3.0, 1.0, 1.0), (0.5, 3e3, 1 / 3e3), (0.5, 1e-3, 1.0), (1.0, 1.0, 40.0),
                                    (0.5, 1.0, 1e-4)):
        w = workloads.make_workload("norms", num_q_heads=8, num_kv_heads=2, seq_lens=[150, 40], seed=13,
                                    dtype=np.float32, lognormal_sigma=sigma)
        codec = oracle.OracleCodec(128, 42)
        kraw = w.rows("k") * np.float32(scale_raw)
        vraw = w.rows("v") * np.float32(scale_raw)
        kp, _ = codec.write_kv(kraw, w.zero_pages(4), w.slots, 4)
        vp, _ = codec.write_kv(vraw, w.zero_pages(4), w.slots, 4)
        q = w.queries() * np.float32(q_mul)
        ref = oracle.paged_decode(q, kp, vp, w.block_table, w.seq_lens, 4, 4, codec.signs,
                                  codec.centroids32(4), codec.centroids32(4))
        out = _decode(ctx, w, torch.from_numpy(q).cuda(), torch.from_numpy(kp).cuda(),
                      torch.from_numpy(vp).cuda())
        # compare relative to the output scale
        s = float(np.abs(ref).max()) or 1.0
        r = compare_decode(out / s, ref / s, f"norms sigma={sigma} x{scale_raw} q*{q_mul}")
        print(f"  norms sigma={sigma} x{scale_raw} q*{q_mul}: {r}", flush=True)


def test_repeated_calls_are_deterministic(ctx):
    w = workloads.make_workload("det", num_q_heads=16, num_kv_heads=2, seq_lens=[700, 300], seed=14)
    codec, _, _, kp, vp = _oracle_pipeline(w)
    q = torch.from_numpy(w.queries()).cuda()
    kpt, vpt = torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda()
    a = _decode(ctx, w, q, kpt, vpt)
    b = _decode(ctx, w, q, kpt, vpt)
    assert np.array_equal(a, b)


def test_out_of_range_block_ids_and_lengths(ctx):
    # Block ids outside [0, num_blocks) read as zero rows, and a device length
    # beyond the block table is clamped to it.  The page tensors are views into
    # larger buffers whose extra pages hold 0xFF bytes, and the workspace has
    # slack, so even an unbounded read would stay inside allocated memory (and
    # show up as a mismatch, not a fault).
    w = workloads.make_workload("bounds", num_q_heads=8, num_kv_heads=2, seq_lens=[100, 40], seed=21)
    print(f"[decode] bounds B={w.batch} lens={w.seq_lens.tolist()} table={w.block_table.shape}", flush=True)
    codec, _, _, kp, vp = _oracle_pipeline(w)
    NB = kp.shape[0]
    max_blocks = w.block_table.shape[1]
    bt = w.block_table.copy()
    bt[0, 2] = NB       # one past the end
    bt[0, 4] = -2       # negative
    dev_lens = np.array([100, 40 + 10000], dtype=np.int32)
    # reference: the two bad ids point at appended zero pages; length 1 clamped
    zero = np.zeros((2,) + kp.shape[1:], dtype=np.uint8)
    bt_ref = bt.copy()
    bt_ref[0, 2], bt_ref[0, 4] = NB, NB + 1
    ref_lens = np.array([100, max_blocks * w.block_size], dtype=np.int32)
    q = w.queries()
    ref = oracle.paged_decode(q, np.concatenate([kp, zero]), np.concatenate([vp, zero]), bt_ref, ref_lens,
                              w.k_bits, w.v_bits, codec.signs, codec.centroids32(w.k_bits),
                              codec.centroids32(w.v_bits))
    pages = []
    for p in (kp, vp):
        big = torch.full((NB + 3,) + p.shape[1:], 0xFF, dtype=torch.uint8, device="cuda")
        big[2:2 + NB] = torch.from_numpy(p).cuda()
        pages.append(big[2:2 + NB])
    need = api.decode_workspace_bytes(ctx, w.batch, w.num_q_heads, w.num_kv_heads, max_blocks * w.block_size)
    ws = torch.zeros(need + (1 << 16), dtype=torch.uint8, device="cuda")
    out = api.paged_decode(ctx, torch.from_numpy(q).cuda(), pages[0], pages[1], torch.from_numpy(bt).cuda(),
                           torch.from_numpy(dev_lens).cuda(), w.k_bits, w.v_bits,
                           max_seq_len=max_blocks * w.block_size, workspace=ws)
    torch.cuda.synchronize()
    r = compare_decode(out.cpu().numpy(), ref, "bounded block ids and lengths")
    print(f"  max|d| relL2 {r}", flush=True)


def test_long_sequence_max_splits(ctx):
    # one 65547-token sequence (4097 pages): the plan's maximum of 64 splits,
    # 65 pages each and 2 in the last, with a ragged last page
    w = workloads.make_workload("long1", num_q_heads=8, num_kv_heads=1, seq_lens=[65536 + 11], seed=23)
    _run(ctx, w)
