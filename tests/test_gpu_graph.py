"""The write and decode calls inside a captured HIP graph.

The library never allocates and never synchronises inside tq_write_kv_pair
and tq_paged_decode (the caller owns out, the workspace and err_count), so a
decode step can be captured once and replayed ("vLLM Usage", Live Backend
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
