"""Page pools past 4 GiB: every kernel addresses pages with 64-bit offsets.

A small seeded workload keeps its page table but its pages move up by a
fixed number of blocks, chosen so that they straddle the 2^32-byte mark of
a pool a little over 4 GiB (one pool for K, one for V): some pages sit
below that mark, the rest above it, all of them above 2^31.  On such pools:

* the GPU writers' rows (the K/V pair writer and the single-component
  writer) are the oracle's encoding byte for byte, up to the usual
  near-boundary index exemption;
* the decode (staged kernel with 8 KV heads, wave kernel with 2) and a
  causal chunk of up to 8 queries per sequence match the oracle's over the
  unmoved pages (2e-3 max-abs, 1e-3 rel-L2);
* the dense readback at the moved slots matches the oracle's reconstruction;
* the prod writer and the prod scores match the oracle's.

Only the moved pages are copied back to the host.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import api, workloads
from tests.parity import compare_decode, compare_pages
from tests.test_gpu_decompress import _norms
from tests.test_gpu_qjl import _check_scores, _compare_rows

pytestmark = pytest.mark.gpu

_MARK = 1 << 32  # bytes


@pytest.fixture(scope="module")
def ctx():
    return api.Context(128, 42)


def _offset(page_bytes: int, num_blocks: int) -> int:
    """Block shift that puts the middle of num_blocks pages at the 2^32-byte mark."""
    off = _MARK // page_bytes - num_blocks // 2
    assert off * page_bytes > (1 << 31) and (off + num_blocks) * page_bytes > _MARK
    return off


def _moved(w, off):
    """Block table and slots of w with every page id raised by off."""
    bt = w.block_table.astype(np.int64) + off
    assert bt.max() < np.iinfo(np.int32).max
    slots = np.where(w.slots >= 0, w.slots + off * w.block_size, -1).astype(np.int64)
    return bt.astype(np.int32), slots


@pytest.mark.parametrize("hkv,kernel", [(8, "staged"), (2, "wave")])
def test_write_decode_readback_past_4gib(ctx, hkv, kernel):
    w = workloads.make_workload(f"big{hkv}", num_q_heads=8 * hkv, num_kv_heads=hkv, seq_lens=[700, 33, 1500, 0],
                                seed=70 + hkv, outlier_frac=0.02)
    assert api.decode_kernel(w.batch, w.num_q_heads, hkv, w.max_seq_len, w.k_bits, w.v_bits) == kernel
    shape = w.page_shape(w.k_bits)
    page_bytes = int(np.prod(shape[1:]))
    off = _offset(page_bytes, w.num_blocks)
    NB = off + w.num_blocks
    print(f"[bigpool] Hkv={hkv} {kernel}: pool {NB} pages x {page_bytes} B = {NB * page_bytes / 2**30:.2f} GiB, "
          f"pages {off}..{NB - 1}", flush=True)
    codec = oracle.OracleCodec(128, w.rht_seed)
    kraw, vraw = w.rows("k"), w.rows("v")
    kp, near_k = codec.write_kv(kraw, w.zero_pages(w.k_bits), w.slots, w.k_bits)
    vp, near_v = codec.write_kv(vraw, w.zero_pages(w.v_bits), w.slots, w.v_bits)
    q = w.queries()
    ref = oracle.paged_decode(q, kp, vp, w.block_table, w.seq_lens, w.k_bits, w.v_bits, codec.signs,
                              codec.centroids32(w.k_bits), codec.centroids32(w.v_bits))

    bt, slots = _moved(w, off)
    kbig = torch.zeros((NB,) + tuple(shape[1:]), dtype=torch.uint8, device="cuda")
    vbig = torch.zeros((NB,) + tuple(w.page_shape(w.v_bits)[1:]), dtype=torch.uint8, device="cuda")
    slots_d = torch.from_numpy(slots).cuda()
    kraw_d, vraw_d = torch.from_numpy(kraw).cuda(), torch.from_numpy(vraw).cuda()
    api.write_kv_pair(ctx, kraw_d, vraw_d, kbig, vbig, slots_d, w.k_bits, w.v_bits)
    torch.cuda.synchronize()
    written = int((w.slots >= 0).sum()) * hkv
    compare_pages(kbig[off:].cpu().numpy(), kp, near_k, w.k_bits, written)
    compare_pages(vbig[off:].cpu().numpy(), vp, near_v, w.v_bits, written)
    assert not kbig[:off].any() and not vbig[:off].any()  # nothing below the moved pages

    out = api.paged_decode(ctx, torch.from_numpy(q).cuda(), kbig, vbig, torch.from_numpy(bt).cuda(),
                           torch.from_numpy(w.seq_lens).cuda(), w.k_bits, w.v_bits, max_seq_len=w.max_seq_len)
    torch.cuda.synchronize()
    r = compare_decode(out.cpu().numpy(), ref, f"decode past 4 GiB ({kernel})")
    print(f"  decode max|d| relL2 {r}", flush=True)

    # a causal chunk of up to 8 queries per sequence over the same pages (its
    # prefix decode and the readback of the chunk's own rows)
    ql, Lq = [8, 5, 1, 0], 8
    qc = np.random.default_rng(hkv).standard_normal((w.batch, Lq, w.num_q_heads, 128), dtype=np.float32)
    qc = qc.astype(np.float16)
    ref_c = oracle.paged_prefill(qc.astype(np.float32), np.array(ql), kp, vp, w.block_table, w.seq_lens, w.k_bits,
                                 w.v_bits, codec.signs, codec.centroids32(w.k_bits), codec.centroids32(w.v_bits))
    out_c = api.paged_prefill(ctx, torch.from_numpy(qc).cuda(), torch.tensor(ql, dtype=torch.int32).cuda(), kbig, vbig,
                              torch.from_numpy(bt).cuda(), torch.from_numpy(w.seq_lens).cuda(), w.k_bits, w.v_bits)
    torch.cuda.synchronize()
    r = compare_decode(out_c.cpu().numpy().reshape(-1, w.num_q_heads, 128), ref_c.reshape(-1, w.num_q_heads, 128),
                       "multi-query past 4 GiB")
    print(f"  multi-query max|d| relL2 {r}", flush=True)

    # the single-component writer over the same rows rewrites the same bytes
    kbig[off:].zero_()
    api.write_kv(ctx, kraw_d, kbig, slots_d, w.k_bits)
    torch.cuda.synchronize()
    compare_pages(kbig[off:].cpu().numpy(), kp, near_k, w.k_bits, written)

    # readback at the moved slots, against the oracle's reconstruction of the
    # oracle's rows (rows with an exempt index mismatch left out)
    got = api.decompress_kv(ctx, kbig, slots_d, w.k_bits).cpu().numpy().astype(np.float64)
    rb = codec.decompress_kv(kp, w.slots, w.k_bits)
    gk = kbig[off:].cpu().numpy()
    s = w.slots
    same = np.all(gk[s // 16, s % 16] == kp[s // 16, s % 16], axis=-1)  # [N, Hkv]
    assert same.mean() > 0.99
    n = _norms(kp, s)
    d = np.abs(got - rb)[same]
    assert (d <= 4e-6 * n[same][:, None] + 2.0 ** -24 * np.abs(rb[same])).all(), float(d.max())


def test_prod_codec_past_4gib(ctx):
    bits, hkv, G = 4, 2, 8
    w = workloads.make_workload("bigprod", num_q_heads=hkv * G, num_kv_heads=hkv, seq_lens=[600, 45, 1200],
                                seed=81, outlier_frac=0.02)
    RB = oracle.prod_row_bytes(128, bits)
    page_bytes = 16 * hkv * RB
    off = _offset(page_bytes, w.num_blocks)
    NB = off + w.num_blocks
    print(f"[bigpool] prod K{bits}: pool {NB} pages x {page_bytes} B = {NB * page_bytes / 2**30:.2f} GiB", flush=True)
    S = workloads.qjl_matrix(128, seed=9)
    signs = oracle.rht_signs(42, 128)
    ref_pages, near_i, near_s = oracle.write_prod(w.rows("k"), np.zeros((w.num_blocks, 16, hkv, RB), np.uint8),
                                                  w.slots, bits, signs, S)
    bt, slots = _moved(w, off)
    big = torch.zeros((NB, 16, hkv, RB), dtype=torch.uint8, device="cuda")
    S_d = torch.from_numpy(S).cuda()
    api.write_kv_prod(ctx, torch.from_numpy(w.rows("k")).cuda(), big, torch.from_numpy(slots).cuda(), bits, S_d)
    torch.cuda.synchronize()
    got_pages = big[off:].cpu().numpy()
    assert not big[:off].any()
    keep = w.slots[w.slots >= 0]
    _compare_rows(got_pages[keep // 16, keep % 16], ref_pages[keep // 16, keep % 16],
                  near_i[keep // 16, keep % 16], near_s[keep // 16, keep % 16], bits, "prod writer past 4 GiB")

    # scores over the GPU's rows against the oracle's estimator over the
    # oracle's rows; scores of rows whose bytes carry an exempt mismatch
    # (index or sign) are left out
    q = w.queries()
    ref = oracle.paged_prod_scores(q, ref_pages, w.block_table, w.seq_lens, bits, signs, S)
    got = api.prod_scores(ctx, torch.from_numpy(q).cuda(), big, torch.from_numpy(bt).cuda(),
                          torch.from_numpy(w.seq_lens).cuda(), bits, S_d)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    norms = np.zeros(ref.shape)
    mask = np.zeros(ref.shape, bool)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        t = np.arange(L)
        gi, _, gz, _ = oracle.prod_bytes_to_rows(got_pages[w.block_table[b, t // 16], t % 16], bits, 128)
        ri, rn, rz, _ = oracle.prod_bytes_to_rows(ref_pages[w.block_table[b, t // 16], t % 16], bits, 128)
        same = np.all(gi == ri, axis=-1) & np.all(gz == rz, axis=-1)  # [L, Hkv]
        mask[b, :, :L] = np.repeat(same.T, G, axis=0)
        norms[b, :, :L] = np.repeat(rn.astype(np.float64).T, G, axis=0)
    assert mask.sum() > 0.99 * sum(int(L) for L in w.seq_lens) * w.num_q_heads
    _check_scores(np.where(mask, got, 0.0), np.where(mask, ref, 0.0), q, norms, "prod scores past 4 GiB")
