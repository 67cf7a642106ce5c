"""The library's calls inside a captured HIP graph.

The library never allocates and never synchronises inside tq_write_kv_pair,
tq_paged_decode and tq_paged_decode_append (the caller owns out, the
workspace and err_count), so a decode step can be captured once and replayed ("vLLM Usage", Live Backend
Gap: graph buffer ownership).  The graph holds only the library's kernels: the
error counter is zeroed before the capture, so no memset is recorded.  Every
replay, with eager work and synchronisations between replays, must give the
eager call's output bit for bit.
"""

import numpy as np
import pytest
import torch

from paged_decode_attention_tq_amd import api, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    return api.Context(128, 42)


# wave-private split over workgroups (with its merge kernel; the second case
# with an empty sequence), wave-private as one workgroup (no merge kernel),
# staged
@pytest.mark.parametrize("hkv,G,lens", [(2, 8, [2100, 33, 1500]), (2, 8, [700, 33, 0]), (1, 2, [64, 17, 0]),
                                        (8, 8, [700, 33, 1500])])
def test_graph_replays_equal_eager(ctx, hkv, G, lens):
    w = workloads.make_workload(f"graph{hkv}", num_q_heads=hkv * G, num_kv_heads=hkv, seq_lens=lens, seed=40 + hkv)
    kernel = api.decode_kernel(w.batch, w.num_q_heads, hkv, w.max_seq_len, 4, 4)
    print(f"[graph] Hkv={hkv} G={G} lens={w.seq_lens.tolist()} kernel={kernel}", flush=True)
    dev = torch.device("cuda")
    kp = torch.zeros(w.page_shape(4), dtype=torch.uint8, device=dev)
    vp = torch.zeros(w.page_shape(4), dtype=torch.uint8, device=dev)
    slots = torch.from_numpy(w.slots).to(dev)
    kraw = torch.from_numpy(w.rows("k")).to(dev)
    vraw = torch.from_numpy(w.rows("v")).to(dev)
    api.write_kv_pair(ctx, kraw, vraw, kp, vp, slots, 4, 4)
    # the step: rewrite the last token of every non-empty sequence, then decode
    last = torch.from_numpy((w.cu_seqlens[1:] - 1)[w.seq_lens > 0].astype(np.int64)).to(dev)
    new_slots = slots[last].contiguous()
    k_new, v_new = kraw[last].contiguous(), vraw[last].contiguous()
    q = torch.from_numpy(w.queries()).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(api.decode_workspace_bytes(ctx, w.batch, w.num_q_heads, hkv, w.max_seq_len), dtype=torch.uint8,
                     device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def step():
        api.write_kv_pair(ctx, k_new, v_new, kp, vp, new_slots, 4, 4, err_count=err, check_slots=False)
        api.paged_decode(ctx, q, kp, vp, bt, lens, 4, 4, max_seq_len=w.max_seq_len, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    assert int(err.item()) == 0

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))  # eager work between replays
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"
        del junk
    assert int(err.item()) == 0


def test_graph_readback_hybrid_and_multi_query(ctx):
    # the other entry points allocate nothing and never synchronise either:
    # readback + hybrid decode + multi-query attention captured together,
    # every replay equal to the eager calls bit for bit
    w = workloads.make_workload("graphx", num_q_heads=16, num_kv_heads=2, seq_lens=[700, 33, 150], seed=44)
    print(f"[graph] readback + hybrid + multi-query lens={w.seq_lens.tolist()}", flush=True)
    dev = torch.device("cuda")
    kp = torch.zeros(w.page_shape(4), dtype=torch.uint8, device=dev)
    vp = torch.zeros(w.page_shape(4), dtype=torch.uint8, device=dev)
    slots = torch.from_numpy(w.slots).to(dev)
    api.write_kv_pair(ctx, torch.from_numpy(w.rows("k")).to(dev), torch.from_numpy(w.rows("v")).to(dev), kp, vp,
                      slots, 4, 4)
    bt = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    q = torch.from_numpy(w.queries()).to(dev)
    rl = np.array([16, 0, 5], dtype=np.int32)
    rk, rv = w.recent_window(16, rl, seed=3)
    rk, rv, rl = torch.from_numpy(rk).to(dev), torch.from_numpy(rv).to(dev), torch.from_numpy(rl).to(dev)
    Lq = 4
    pq = torch.randn((w.batch, Lq, w.num_q_heads, 128), device=dev).to(torch.float16)
    ql = torch.tensor([4, 2, 1], dtype=torch.int32, device=dev)
    dense = torch.empty((w.num_tokens, 2, 128), dtype=torch.float16, device=dev)
    hout = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=dev)
    pout = torch.empty((w.batch, Lq, w.num_q_heads, 128), dtype=torch.float32, device=dev)
    hws = torch.empty(api.hybrid_workspace_bytes(ctx, w.batch, w.num_q_heads, 2, w.max_seq_len), dtype=torch.uint8,
                      device=dev)
    pws = torch.empty(api.prefill_workspace_bytes(ctx, w.batch, Lq, w.num_q_heads, 2, w.max_seq_len),
                      dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def step():
        api.decompress_kv(ctx, kp, slots, 4, out=dense, err_count=err, check_slots=False)
        api.paged_decode_hybrid(ctx, q, kp, vp, bt, lens, rk, rv, rl, 4, 4, max_seq_len=w.max_seq_len, out=hout,
                                workspace=hws)
        api.paged_prefill(ctx, pq, ql, kp, vp, bt, lens, 4, 4, max_seq_len=w.max_seq_len, out=pout, workspace=pws)

    step()
    torch.cuda.synchronize()
    eager = [dense.clone(), hout.clone(), pout.clone()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for t in (dense, hout, pout):
            t.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((dense, hout, pout), eager):
            assert torch.equal(got, want), f"replay {r} differs from the eager call"
        del junk
    assert int(err.item()) == 0


def test_graph_prod_codec(ctx):
    # the prod key codec's writer and scores captured together: every replay
    # (pages cleared and scores overwritten in between) equal to the eager
    # calls bit for bit
    w = workloads.make_workload("graphp", num_q_heads=16, num_kv_heads=2, seq_lens=[700, 33, 150], seed=45)
    print(f"[graph] prod writer + scores lens={w.seq_lens.tolist()}", flush=True)
    dev = torch.device("cuda")
    bits = 4
    pages = torch.zeros((w.num_blocks, 16, 2, api.prod_row_bytes(128, bits)), dtype=torch.uint8, device=dev)
    slots = torch.from_numpy(w.slots).to(dev)
    raw = torch.from_numpy(w.rows("k")).to(dev)
    S = torch.from_numpy(workloads.qjl_matrix(128, seed=5)).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    q = torch.from_numpy(w.queries()).to(dev)
    scores = torch.empty((w.batch, w.num_q_heads, w.max_seq_len), dtype=torch.float32, device=dev)
    ws = torch.empty(api.prod_scores_workspace_bytes(w.batch, w.num_q_heads), dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def step():
        api.write_kv_prod(ctx, raw, pages, slots, bits, S, err_count=err, check_slots=False)
        api.prod_scores(ctx, q, pages, bt, lens, bits, S, max_seq_len=w.max_seq_len, out=scores, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [pages.clone(), scores.clone()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        pages.zero_()
        scores.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((pages, scores), eager):
            assert torch.equal(got, want), f"replay {r} differs from the eager call"
        del junk
    assert int(err.item()) == 0


# the one-call decode step: the staged kernel's appending instantiation, and a
# wave-kernel shape (writer launch, then the decode and its merge)
@pytest.mark.parametrize("hkv,G,lens", [(8, 8, [700, 33, 1500]), (2, 8, [700, 33, 0])])
def test_graph_append_step(ctx, hkv, G, lens):
    w = workloads.make_workload(f"grapp{hkv}", num_q_heads=hkv * G, num_kv_heads=hkv, seq_lens=lens, seed=60 + hkv)
    kernel = api.decode_kernel(w.batch, w.num_q_heads, hkv, w.max_seq_len, 4, 4)
    print(f"[graph] append Hkv={hkv} G={G} lens={w.seq_lens.tolist()} kernel={kernel}", flush=True)
    dev = torch.device("cuda")
    kp = torch.zeros(w.page_shape(4), dtype=torch.uint8, device=dev)
    vp = torch.zeros(w.page_shape(4), dtype=torch.uint8, device=dev)
    kraw = torch.from_numpy(w.rows("k")).to(dev)
    vraw = torch.from_numpy(w.rows("v")).to(dev)
    api.write_kv_pair(ctx, kraw, vraw, kp, vp, torch.from_numpy(w.slots).to(dev), 4, 4)
    # the new rows: every non-empty sequence's last token (zeros for an empty one)
    has = torch.from_numpy(w.seq_lens > 0).to(dev)
    last = torch.from_numpy(np.maximum(w.cu_seqlens[1:] - 1, 0).astype(np.int64)).to(dev)
    k_new = torch.where(has[:, None, None], kraw[last], torch.zeros_like(kraw[last])).contiguous()
    v_new = torch.where(has[:, None, None], vraw[last], torch.zeros_like(vraw[last])).contiguous()
    q = torch.from_numpy(w.queries()).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(api.decode_workspace_bytes(ctx, w.batch, w.num_q_heads, hkv, w.max_seq_len), dtype=torch.uint8,
                     device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def step():
        api.paged_decode_append(ctx, q, k_new, v_new, kp, vp, bt, lens, 4, 4, max_seq_len=w.max_seq_len, out=out,
                                workspace=ws, err_count=err, check_pages=False)

    step()
    torch.cuda.synchronize()
    eager, kp_eager, vp_eager = out.clone(), kp.clone(), vp.clone()
    assert int(err.item()) == 0

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))  # eager work between replays
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"
        assert torch.equal(kp, kp_eager) and torch.equal(vp, vp_eager), f"replay {r}: pages differ"
        del junk
    assert int(err.item()) == 0
