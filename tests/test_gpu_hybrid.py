"""GPU parity of the hybrid decode (tq_paged_decode_hybrid) against the oracle.

Packed history (pages written by the oracle writer, and at full size by the
GPU writer with the pages byte-checked elsewhere) plus an exact recent window
of K/V rows; the oracle attends over both with one softmax in float64.
Tolerance as the decode's: max-abs 2e-3 and relative L2 1e-3.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import api, workloads
from tests.oracle_par import sequence_hybrid_outputs, sequence_pages
from tests.parity import compare_decode

pytestmark = pytest.mark.gpu

_TORCH = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def ctx():
    return api.Context(128, 42)


def _window(w, cap, rl, dt, seed):
    rk, rv = w.recent_window(cap, rl, seed=seed)
    tk = torch.from_numpy(rk.astype(np.float32)).to(_TORCH[dt])
    tv = torch.from_numpy(rv.astype(np.float32)).to(_TORCH[dt])
    # the oracle takes the values the kernel reads (bf16 rounding included)
    return tk, tv, tk.float().numpy(), tv.float().numpy()


# (KV heads, group, lengths, window lengths, window capacity): the wave kernel,
# the wave kernel as one workgroup, the staged kernel; empty history, empty
# window, both empty, windows across the 64-token rounds, group > 8
CASES = [
    (2, 8, [300, 0, 45, 0, 129], [7, 33, 0, 0, 130], 130),
    (1, 2, [64, 17, 0], [64, 65, 1], 65),
    (8, 8, [700, 33, 1500], [128, 1, 0], 128),
    (2, 12, [90, 16], [20, 64], 64),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("dt", ["fp16", "bf16", "fp32"])
def test_hybrid_matches_oracle(ctx, case, dt):
    hkv, G, lens, rl, cap = CASES[case]
    w = workloads.make_workload(f"hyb{case}", num_q_heads=hkv * G, num_kv_heads=hkv, seq_lens=lens,
                                seed=70 + case, lognormal_sigma=0.5)
    kernel = api.decode_kernel(w.batch, w.num_q_heads, hkv, max(1, w.max_seq_len), 4, 4)
    print(f"[hybrid] case {case} {dt} Hkv={hkv} G={G} lens={lens} window={rl} cap={cap} kernel={kernel}", flush=True)
    codec = oracle.OracleCodec(128, 42)
    kp, _ = codec.write_kv(w.rows("k"), w.zero_pages(4), w.slots, 4)
    vp, _ = codec.write_kv(w.rows("v"), w.zero_pages(4), w.slots, 4)
    tk, tv, rk, rv = _window(w, cap, rl, dt, seed=case)
    q = w.queries()
    ref = oracle.paged_decode_hybrid(q, kp, vp, w.block_table, w.seq_lens, rk, rv, np.array(rl), 4, 4,
                                     codec.signs, codec.centroids32(4), codec.centroids32(4))
    out = api.paged_decode_hybrid(ctx, torch.from_numpy(q).cuda(), torch.from_numpy(kp).cuda(),
                                  torch.from_numpy(vp).cuda(), torch.from_numpy(w.block_table).cuda(),
                                  torch.from_numpy(w.seq_lens).cuda(), tk.cuda(), tv.cuda(),
                                  torch.tensor(rl, dtype=torch.int32).cuda(), 4, 4, max_seq_len=max(1, w.max_seq_len))
    torch.cuda.synchronize()
    res = compare_decode(out.cpu().numpy(), ref, f"hybrid case {case} {dt}")
    print(f"  max|d| relL2 {res}", flush=True)


def test_empty_window_equals_the_decode(ctx):
    # recent_cap 0: exactly tq_paged_decode, bit for bit
    w = workloads.make_workload("hyb_empty", num_q_heads=16, num_kv_heads=2, seq_lens=[300, 45, 0], seed=5)
    print("[hybrid] cap 0 against the plain decode", flush=True)
    codec = oracle.OracleCodec(128, 42)
    kp = torch.from_numpy(codec.write_kv(w.rows("k"), w.zero_pages(4), w.slots, 4)[0]).cuda()
    vp = torch.from_numpy(codec.write_kv(w.rows("v"), w.zero_pages(4), w.slots, 4)[0]).cuda()
    q = torch.from_numpy(w.queries()).cuda()
    bt, lens = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    a = api.paged_decode(ctx, q, kp, vp, bt, lens, 4, 4)
    z = torch.zeros((w.batch, 0, 2, 128), dtype=torch.float16, device="cuda")
    b = api.paged_decode_hybrid(ctx, q, kp, vp, bt, lens, z, z, torch.zeros(w.batch, dtype=torch.int32).cuda(), 4, 4)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["long_context", "ragged_write"])
def test_full_size_sampled(ctx, name):
    # every row written by the GPU writer at the configuration's full size, a
    # 128-row fp16 window per sequence (seeded lengths 0..128), one hybrid
    # call; the longest and the shortest sequence checked on all query heads
    w = workloads.preset(name)
    cap = 128
    rl = np.random.default_rng(9).integers(0, cap + 1, size=w.batch)
    print(f"[hybrid] full size {name}: B={w.batch} tokens={w.num_tokens} window cap {cap}", flush=True)
    dev = torch.device("cuda")
    ctx_pages = {}
    for comp, bits in (("k", w.k_bits), ("v", w.v_bits)):
        pg = torch.zeros(w.page_shape(bits), dtype=torch.uint8, device=dev)
        raw = torch.from_numpy(w.rows(comp, threads=16)).to(dev)
        api.write_kv(ctx, raw, pg, torch.from_numpy(w.slots).to(dev), bits)
        del raw
        ctx_pages[comp] = pg
    tk, tv, rk, rv = _window(w, cap, rl, "fp16", seed=11)
    q = w.queries()
    out = api.paged_decode_hybrid(ctx, torch.from_numpy(q).to(dev), ctx_pages["k"], ctx_pages["v"],
                                  torch.from_numpy(w.block_table).to(dev), torch.from_numpy(w.seq_lens).to(dev),
                                  tk.to(dev), tv.to(dev), torch.from_numpy(rl.astype(np.int32)).to(dev),
                                  w.k_bits, w.v_bits, max_seq_len=w.max_seq_len)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    order = np.argsort(w.seq_lens, kind="stable")
    for b in sorted({int(order[0]), int(order[-1])}):
        kpo, _, _ = sequence_pages(codec, w, b, "k", w.k_bits)
        vpo, _, _ = sequence_pages(codec, w, b, "v", w.v_bits)
        ref = sequence_hybrid_outputs(codec, w, b, kpo, vpo, q, rk[b], rv[b], int(rl[b]))
        res = compare_decode(out[b], ref, f"{name} hybrid sequence {b}")
        print(f"  seq {b} ({w.seq_lens[b]} tokens + {rl[b]} window rows): max|d| relL2 {res}", flush=True)
