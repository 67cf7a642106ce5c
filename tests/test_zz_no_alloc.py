"""The allocation-free decode entry point against the workspace one.

tq_paged_decode_noalloc runs the same kernels with the library's static
scratch in place of a caller workspace, so its outputs must equal
tq_paged_decode's bit for bit: checked on two calls in a row, the second with
a smaller input (the scratch keeps the first call's partials), on the
wave-private and the staged decode kernels.  Sizes whose partials exceed the
scratch are refused before any launch.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import api, workloads
from tests.parity import compare_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    return api.Context(128, 42)


def _inputs(w):
    codec = oracle.OracleCodec(128, 42)
    kp, _ = codec.write_kv(w.rows("k"), w.zero_pages(w.k_bits), w.slots, w.k_bits)
    vp, _ = codec.write_kv(w.rows("v"), w.zero_pages(w.v_bits), w.slots, w.v_bits)
    dev = torch.device("cuda")
    t = dict(q=torch.from_numpy(w.queries()).to(dev), kp=torch.from_numpy(kp).to(dev), vp=torch.from_numpy(vp).to(dev),
             bt=torch.from_numpy(w.block_table).to(dev), lens=torch.from_numpy(w.seq_lens).to(dev))
    ref = oracle.paged_decode(w.queries(), kp, vp, w.block_table, w.seq_lens, w.k_bits, w.v_bits, codec.signs,
                              codec.centroids32(w.k_bits), codec.centroids32(w.v_bits))
    return t, ref


@pytest.mark.parametrize("hkv", [2, 8])  # wave-private and staged decode kernels
def test_noalloc_equals_workspace_entry_point_on_two_calls(ctx, hkv):
    big = workloads.make_workload(f"na_big{hkv}", num_q_heads=8 * hkv, num_kv_heads=hkv, seq_lens=[3000, 5000, 17, 1],
                                  seed=50 + hkv)
    small = workloads.make_workload(f"na_small{hkv}", num_q_heads=4 * hkv, num_kv_heads=hkv, seq_lens=[300, 9],
                                    seed=60 + hkv)
    for w in (big, small):
        print(f"[noalloc] Hkv={hkv} lens={w.seq_lens.tolist()} kernel="
              f"{api.decode_kernel(w.batch, w.num_q_heads, hkv, w.max_seq_len, 4, 4)}", flush=True)
        t, ref = _inputs(w)
        a = api.paged_decode_noalloc(ctx, t["q"], t["kp"], t["vp"], t["bt"], t["lens"], 4, 4, max_seq_len=w.max_seq_len)
        b = api.paged_decode(ctx, t["q"], t["kp"], t["vp"], t["bt"], t["lens"], 4, 4, max_seq_len=w.max_seq_len)
        torch.cuda.synchronize()
        assert torch.equal(a, b), "the allocation-free call differs from the workspace call"
        compare_decode(a.cpu().numpy(), ref, f"noalloc Hkv={hkv}")


def test_noalloc_refuses_sizes_beyond_the_scratch(ctx):
    # 4096 sequences x 64 query heads need far more than the 32 MiB of partials;
    # the call is refused before any pointer is touched
    need = api.decode_workspace_bytes(ctx, 4096, 64, 8, 131072)
    assert need > (32 << 20)
    dev = torch.device("cuda")
    q = torch.zeros((4096, 64, 128), dtype=torch.float16, device=dev)
    pages = torch.zeros((1, 16, 8, 68), dtype=torch.uint8, device=dev)
    bt = torch.zeros((4096, 8192), dtype=torch.int32, device=dev)
    lens = torch.zeros(4096, dtype=torch.int32, device=dev)
    with pytest.raises(api.TQError, match="workspace too small"):
        api.paged_decode_noalloc(ctx, q, pages, pages, bt, lens, 4, 4, max_seq_len=131072)
