"""GPU parity of the appending decode (tq_paged_decode_append).

One call writes every sequence's new K and V row (its last token) and
decodes.  Each case checks it bit for bit against the two-call path on the
same inputs (tq_write_kv_pair at the last tokens' slots, then
tq_paged_decode): equal page bytes everywhere and equal outputs.  It also
checks it against the oracle (its writer over every token, its decode) to
the decode tolerance (2e-3 max-abs, 1e-3 rel-L2).  The cases cover:

* the staged kernel, with every KV head in one workgroup and with the heads
  split over workgroups;
* the wave kernel with 2 and 4 KV heads, and its one-workgroup launch;
* new rows in fp32, fp16 and bf16;
* sequences that end on a page's last row and on a page's first row, and an
  empty sequence;
* a last page whose block id lies outside the pages (counted, not written);
* the full long-context workload against the two-call path.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import api, workloads
from tests.parity import compare_decode

pytestmark = pytest.mark.gpu

_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def ctx():
    return api.Context(128, 42)


def _split(w):
    """Flat indices of every sequence's last token (-1 for an empty sequence)."""
    ends = np.cumsum(w.seq_lens.astype(np.int64)) - 1
    return np.where(w.seq_lens > 0, ends, -1)


def _run(ctx, w, dt, kernel, bad_seq=None):
    kb, vb = w.k_bits, w.v_bits
    got_kernel = api.decode_kernel(w.batch, w.num_q_heads, w.num_kv_heads, w.max_seq_len, kb, vb)
    print(f"[append] {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} K{kb}V{vb} {dt} "
          f"lens={w.seq_lens.tolist()} kernel={got_kernel} bad_seq={bad_seq}", flush=True)
    assert got_kernel == kernel
    last = _split(w)
    has = last >= 0
    kraw, vraw = w.rows("k"), w.rows("v")
    # the new rows in the call's dtype, and the values the GPU reads from them
    k_new = torch.zeros((w.batch, w.num_kv_heads, 128), dtype=_DT[dt])
    v_new = torch.zeros((w.batch, w.num_kv_heads, 128), dtype=_DT[dt])
    k_new[torch.from_numpy(has)] = torch.from_numpy(kraw[last[has]].astype(np.float32)).to(_DT[dt])
    v_new[torch.from_numpy(has)] = torch.from_numpy(vraw[last[has]].astype(np.float32)).to(_DT[dt])
    kfull = kraw.astype(np.float32)
    vfull = vraw.astype(np.float32)
    kfull[last[has]] = k_new[torch.from_numpy(has)].float().numpy()
    vfull[last[has]] = v_new[torch.from_numpy(has)].float().numpy()

    bt = w.block_table.copy()
    if bad_seq is not None:
        L = int(w.seq_lens[bad_seq])
        bt[bad_seq, (L - 1) // 16] = -1
    # history: every token but the last ones, written by the oracle
    codec = oracle.OracleCodec(128, w.rht_seed)
    hist = w.slots.copy()
    hist[last[has]] = -1
    kp, _ = codec.write_kv(kfull, w.zero_pages(kb), hist, kb)
    vp, _ = codec.write_kv(vfull, w.zero_pages(vb), hist, vb)

    q = torch.from_numpy(w.queries()).cuda()
    bt_d = torch.from_numpy(bt).cuda()
    lens_d = torch.from_numpy(w.seq_lens).cuda()
    # two calls: the writer at the last tokens' slots (-1: no row), then the decode
    slot_new = np.full(w.batch, -1, dtype=np.int64)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        if L > 0 and bt[b, (L - 1) // 16] >= 0:
            slot_new[b] = int(bt[b, (L - 1) // 16]) * 16 + (L - 1) % 16
    kp1, vp1 = torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda()
    api.write_kv_pair(ctx, k_new.cuda(), v_new.cuda(), kp1, vp1, torch.from_numpy(slot_new).cuda(), kb, vb)
    out1 = api.paged_decode(ctx, q, kp1, vp1, bt_d, lens_d, kb, vb, max_seq_len=w.max_seq_len)
    # one call
    kp2, vp2 = torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out2 = api.paged_decode_append(ctx, q, k_new.cuda(), v_new.cuda(), kp2, vp2, bt_d, lens_d, kb, vb,
                                   max_seq_len=w.max_seq_len, err_count=err, check_pages=False)
    torch.cuda.synchronize()
    assert int(err.item()) == (0 if bad_seq is None else 1)
    assert torch.equal(kp1, kp2) and torch.equal(vp1, vp2), "pages differ from the two-call path"
    assert torch.equal(out1, out2), "output differs from the two-call path"
    if bad_seq is None:
        # the oracle: its writer over every token, its decode
        kpo, _ = codec.write_kv(kfull, w.zero_pages(kb), w.slots, kb)
        vpo, _ = codec.write_kv(vfull, w.zero_pages(vb), w.slots, vb)
        ref = oracle.paged_decode(w.queries(), kpo, vpo, w.block_table, w.seq_lens, kb, vb, codec.signs,
                                  codec.centroids32(kb), codec.centroids32(vb))
        r = compare_decode(out2.cpu().numpy(), ref, f"append {w.name} {dt}")
        print(f"  max|d| relL2 vs oracle {r}", flush=True)


# (KV heads, group, bits, lengths, kernel): last tokens on a page's last row
# (16), its first row (17, 1) and an empty sequence
CASES = [
    (8, 8, (4, 4), [700, 33, 1500, 0, 16, 17, 1], "staged"),
    (16, 1, (3, 5), [300, 47, 16, 129], "staged"),
    (2, 8, (4, 2), [700, 33, 1500, 0, 16, 17, 1], "wave"),
    (4, 8, (3, 3), [40, 17, 16, 1, 900, 2, 31, 33], "wave"),
    (1, 2, (4, 4), [64, 0, 17], "wave1"),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("dt", ["fp16", "fp32", "bf16"])
def test_append_matches_two_calls_and_oracle(ctx, case, dt):
    hkv, G, (kb, vb), lens, kernel = CASES[case]
    w = workloads.make_workload(f"app{case}", k_bits=kb, v_bits=vb, num_q_heads=hkv * G, num_kv_heads=hkv,
                                seq_lens=lens, seed=140 + case, outlier_frac=0.02)
    _run(ctx, w, dt, kernel)


@pytest.mark.parametrize("hkv,kernel", [(8, "staged"), (2, "wave")])
def test_append_out_of_range_last_page(ctx, hkv, kernel):
    # sequence 1's last page has block id -1: its rows are not written (the
    # count is 1), and the page reads as zero rows in both paths
    w = workloads.make_workload(f"appbad{hkv}", num_q_heads=8 * hkv, num_kv_heads=hkv, seq_lens=[300, 45, 129],
                                seed=150 + hkv)
    _run(ctx, w, "fp16", kernel, bad_seq=1)


def test_append_raises_when_checked(ctx):
    w = workloads.make_workload("appchk", num_q_heads=4, num_kv_heads=2, seq_lens=[20, 5], seed=160)
    bt = w.block_table.copy()
    bt[0, 1] = w.num_blocks + 7  # the last page of sequence 0 is outside the pages
    kp = torch.zeros(w.page_shape(4), dtype=torch.uint8, device="cuda")
    vp = torch.zeros(w.page_shape(4), dtype=torch.uint8, device="cuda")
    new = torch.zeros((2, 2, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(api.TQError):
        api.paged_decode_append(ctx, torch.from_numpy(w.queries()).cuda(), new, new, kp, vp,
                                torch.from_numpy(bt).cuda(), torch.from_numpy(w.seq_lens).cuda(), 4, 4)


def test_append_full_size_long_context(ctx):
    # the long-context workload at full size (8 x 131072 tokens, 8 KV heads):
    # every row but the last tokens' written by the GPU writer, then the step
    # as one call and as two calls on copies of the pages; the pools and the
    # outputs must be equal bit for bit (the oracle side of this path is
    # covered at reduced size above and by the full-size decode tests)
    w = workloads.preset("long_context")
    print(f"[append] full size long_context: {w.num_tokens} tokens x {w.num_kv_heads} heads", flush=True)
    assert api.decode_kernel(w.batch, w.num_q_heads, w.num_kv_heads, w.max_seq_len, 4, 4) == "staged"
    dev = torch.device("cuda")
    kraw = torch.from_numpy(w.rows("k", threads=16)).to(dev)
    vraw = torch.from_numpy(w.rows("v", threads=16)).to(dev)
    last = torch.from_numpy((w.cu_seqlens[1:] - 1).astype(np.int64)).to(dev)
    slots = torch.from_numpy(w.slots).to(dev)
    hist = slots.clone()
    hist[last] = -1
    kp1 = torch.zeros(w.page_shape(4), dtype=torch.uint8, device=dev)
    vp1 = torch.zeros(w.page_shape(4), dtype=torch.uint8, device=dev)
    api.write_kv_pair(ctx, kraw, vraw, kp1, vp1, hist, 4, 4)
    k_new, v_new = kraw[last].contiguous(), vraw[last].contiguous()
    del kraw, vraw
    kp2, vp2 = kp1.clone(), vp1.clone()
    q = torch.from_numpy(w.queries()).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    api.write_kv_pair(ctx, k_new, v_new, kp1, vp1, slots[last].contiguous(), 4, 4)
    out1 = api.paged_decode(ctx, q, kp1, vp1, bt, lens, 4, 4, max_seq_len=w.max_seq_len)
    out2 = api.paged_decode_append(ctx, q, k_new, v_new, kp2, vp2, bt, lens, 4, 4, max_seq_len=w.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(kp1, kp2) and torch.equal(vp1, vp2), "pages differ from the two-call path"
    assert torch.equal(out1, out2), "output differs from the two-call path"
