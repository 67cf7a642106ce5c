"""GPU parity of the multi-query attention (tq_paged_prefill) against the oracle.

Each sequence's last q_lens[b] tokens query the packed pages causally (their
own K/V rows already written).  Pages from the oracle writer (and at full
size from the GPU writer); the oracle attends in float64.  Tolerance as the
decode's: max-abs 2e-3 and relative L2 1e-3, over every query row.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import api, workloads
from tests.oracle_par import sequence_pages, sequence_prefill_outputs
from tests.parity import compare_decode

pytestmark = pytest.mark.gpu

_TORCH = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def ctx():
    return api.Context(128, 42)


def _queries(w, Lq, dt, seed):
    q = torch.from_numpy(np.random.default_rng(seed).standard_normal((w.batch, Lq, w.num_q_heads, 128),
                                                                     dtype=np.float32)).to(_TORCH[dt])
    return q, q.float().numpy()


# (KV heads, group, lengths, query lengths, Lq): the decode of the prefix runs
# on the wave kernel (group x Lq <= 8), as one workgroup, or staged (64 query
# rows per KV head; 12 with a half-filled second query group; 32 with
# prefixes of a few tokens); mixed batches with one-token and empty chunks; a
# chunk of one page and more
CASES = [
    (2, 2, [300, 45, 129, 9], [4, 1, 3, 0], 4),
    (1, 2, [40, 7, 3], [3, 2, 3], 3),
    (2, 8, [700, 33, 1500], [8, 5, 1], 8),
    (4, 4, [64, 200], [16, 1], 16),
    (2, 8, [90, 16, 17], [1, 1, 1], 1),
    (3, 3, [1000, 17, 33], [4, 4, 2], 4),
    (1, 16, [520, 2, 3], [1, 2, 2], 2),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("dt", ["fp16", "bf16", "fp32"])
def test_prefill_matches_oracle(ctx, case, dt):
    hkv, G, lens, ql, Lq = CASES[case]
    w = workloads.make_workload(f"pre{case}", num_q_heads=hkv * G, num_kv_heads=hkv, seq_lens=lens,
                                seed=90 + case, lognormal_sigma=0.5)
    kernel = api.decode_kernel(w.batch, w.num_q_heads * Lq, hkv, w.max_seq_len, 4, 4)
    print(f"[prefill] case {case} {dt} Hkv={hkv} G={G} lens={lens} q_lens={ql} Lq={Lq} prefix kernel={kernel}",
          flush=True)
    codec = oracle.OracleCodec(128, 42)
    kp, _ = codec.write_kv(w.rows("k"), w.zero_pages(4), w.slots, 4)
    vp, _ = codec.write_kv(w.rows("v"), w.zero_pages(4), w.slots, 4)
    tq, q = _queries(w, Lq, dt, case)
    ref = oracle.paged_prefill(q, np.array(ql), kp, vp, w.block_table, w.seq_lens, 4, 4, codec.signs,
                               codec.centroids32(4), codec.centroids32(4))
    out = torch.full((w.batch, Lq, w.num_q_heads, 128), float("nan"), device="cuda")
    api.paged_prefill(ctx, tq.cuda(), torch.tensor(ql, dtype=torch.int32).cuda(), torch.from_numpy(kp).cuda(),
                      torch.from_numpy(vp).cuda(), torch.from_numpy(w.block_table).cuda(),
                      torch.from_numpy(w.seq_lens).cuda(), 4, 4, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b, n in enumerate(ql):
        assert not got[b, n:].any(), f"rows past q_lens[{b}] = {n} are not zero"
    res = compare_decode(got.reshape(-1, w.num_q_heads, 128), ref.reshape(-1, w.num_q_heads, 128),
                         f"prefill case {case} {dt}")
    print(f"  max|d| relL2 {res}", flush=True)


@pytest.mark.parametrize("kb,vb", [(3, 5), (2, 3), (5, 2)])
def test_prefill_multi_query_bit_widths(ctx, kb, vb):
    # 16 query rows per KV head (two query groups) with other K / V index
    # widths: 3- and 5-bit fields straddle bytes and words
    lens, ql, Lq = [300, 90, 47], [4, 3, 1], 4
    w = workloads.make_workload(f"prebits{kb}{vb}", num_q_heads=8, num_kv_heads=2, seq_lens=lens, seed=70 + kb + vb,
                                outlier_frac=0.02)
    print(f"[prefill] multi-query K{kb}/V{vb} lens={lens} q_lens={ql}", flush=True)
    codec = oracle.OracleCodec(128, 42)
    kp, _ = codec.write_kv(w.rows("k"), w.zero_pages(kb), w.slots, kb)
    vp, _ = codec.write_kv(w.rows("v"), w.zero_pages(vb), w.slots, vb)
    tq, q = _queries(w, Lq, "fp16", kb * 10 + vb)
    ref = oracle.paged_prefill(q, np.array(ql), kp, vp, w.block_table, w.seq_lens, kb, vb, codec.signs,
                               codec.centroids32(kb), codec.centroids32(vb))
    out = api.paged_prefill(ctx, tq.cuda(), torch.tensor(ql, dtype=torch.int32).cuda(), torch.from_numpy(kp).cuda(),
                            torch.from_numpy(vp).cuda(), torch.from_numpy(w.block_table).cuda(),
                            torch.from_numpy(w.seq_lens).cuda(), kb, vb)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    res = compare_decode(got.reshape(-1, w.num_q_heads, 128), ref.reshape(-1, w.num_q_heads, 128),
                         f"prefill multi-query K{kb}/V{vb}")
    print(f"  max|d| relL2 {res}", flush=True)


def test_one_query_equals_the_decode(ctx):
    # q_len 1 everywhere: the decode of the same queries, within the decode's tolerance
    w = workloads.make_workload("pre1", num_q_heads=16, num_kv_heads=2, seq_lens=[300, 45, 5], seed=7)
    print("[prefill] one query per sequence against tq_paged_decode", flush=True)
    codec = oracle.OracleCodec(128, 42)
    kp = torch.from_numpy(codec.write_kv(w.rows("k"), w.zero_pages(4), w.slots, 4)[0]).cuda()
    vp = torch.from_numpy(codec.write_kv(w.rows("v"), w.zero_pages(4), w.slots, 4)[0]).cuda()
    q = torch.from_numpy(w.queries()).cuda()
    bt, lens = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    a = api.paged_decode(ctx, q, kp, vp, bt, lens, 4, 4)
    b = api.paged_prefill(ctx, q[:, None].contiguous(), torch.ones(w.batch, dtype=torch.int32).cuda(), kp, vp, bt,
                          lens, 4, 4)
    torch.cuda.synchronize()
    assert float((a - b[:, 0]).abs().max()) < 1e-5


@pytest.mark.parametrize("name,Lq", [("long_context", 8), ("pages_geometry", 4)])
def test_full_size_sampled(ctx, name, Lq):
    # every row written by the GPU writer at full size, then a chunk of Lq
    # queries per sequence (seeded q_lens 1..Lq); two sequences checked on
    # every query row and head
    w = workloads.preset(name)
    ql = np.random.default_rng(3).integers(1, Lq + 1, size=w.batch).astype(np.int32)
    ql[0] = Lq
    print(f"[prefill] full size {name}: B={w.batch} tokens={w.num_tokens} Lq={Lq} q_lens={ql[:8].tolist()}",
          flush=True)
    dev = torch.device("cuda")
    pages = {}
    for comp, bits in (("k", w.k_bits), ("v", w.v_bits)):
        pg = torch.zeros(w.page_shape(bits), dtype=torch.uint8, device=dev)
        raw = torch.from_numpy(w.rows(comp, threads=16)).to(dev)
        api.write_kv(ctx, raw, pg, torch.from_numpy(w.slots).to(dev), bits)
        del raw
        pages[comp] = pg
    tq, q = _queries(w, Lq, "fp16", 5)
    out = api.paged_prefill(ctx, tq.to(dev), torch.from_numpy(ql).to(dev), pages["k"], pages["v"],
                            torch.from_numpy(w.block_table).to(dev), torch.from_numpy(w.seq_lens).to(dev),
                            w.k_bits, w.v_bits, max_seq_len=w.max_seq_len)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    for b in (0, w.batch - 1):
        kpo, _, _ = sequence_pages(codec, w, b, "k", w.k_bits)
        vpo, _, _ = sequence_pages(codec, w, b, "v", w.v_bits)
        ref = sequence_prefill_outputs(codec, w, b, kpo, vpo, q[b], int(ql[b]))
        res = compare_decode(out[b], ref, f"{name} prefill sequence {b}")
        print(f"  seq {b} ({w.seq_lens[b]} tokens, {ql[b]} queries): max|d| relL2 {res}", flush=True)
