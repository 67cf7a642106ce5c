"""GPU parity at the full workload sizes, on sampled outputs.

Every configuration runs at its full size through the GPU path in the
configuration the benchmark times: the row writer encodes every row of every
sequence into the pages (through the flat slots, with dropped slots where the
workload has them), then one decode over all sequences.  The oracle then
recomputes sampled (sequence, query head) outputs one by one from the same
seeded raw rows: it encodes that sequence's rows of the head's KV head with
its own writer (dropped slots stay zero) and decodes them.  Nothing the GPU
produced is fed to the oracle.  Tolerances are those of the decode parity
tests: max-abs 2e-3 and relative L2 1e-3 over the sampled outputs.
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


def _gpu_path(ctx, w):
    """Write every row on the GPU through the flat slots, then decode."""
    dev = torch.device("cuda")
    kp = torch.zeros(w.page_shape(w.k_bits), dtype=torch.uint8, device=dev)
    vp = torch.zeros(w.page_shape(w.v_bits), dtype=torch.uint8, device=dev)
    slots = torch.from_numpy(w.slots).to(dev)
    for comp, pages, bits in (("k", kp, w.k_bits), ("v", vp, w.v_bits)):
        raw = torch.from_numpy(w.rows(comp, threads=16)).to(dev)
        api.write_kv(ctx, raw, pages, slots, bits)  # checked: raises on out-of-range slots
        del raw
    q = torch.from_numpy(w.queries()).to(dev)
    out = api.paged_decode(ctx, q, kp, vp, torch.from_numpy(w.block_table).to(dev),
                           torch.from_numpy(w.seq_lens).to(dev), w.k_bits, w.v_bits, max_seq_len=w.max_seq_len)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle_head(w, codec, b, h, queries):
    """Oracle output of query head h of sequence b, from its own encoding."""
    L = int(w.seq_lens[b])
    d = w.head_dim
    if L == 0:
        return np.zeros(d)
    G = w.num_q_heads // w.num_kv_heads
    g = h // G
    lo = int(w.cu_seqlens[b])
    dropped = w.slots[lo:lo + L] < 0
    mini_slots = np.where(dropped, -1, np.arange(L)).astype(np.int64)
    npg = (L + w.block_size - 1) // w.block_size
    pages = {}
    for comp, bits in (("k", w.k_bits), ("v", w.v_bits)):
        raw = w.seq_rows(comp, b)[:, g:g + 1, :]
        zero = np.zeros((npg, w.block_size, 1, w.row_bytes(bits)), dtype=np.uint8)
        pages[comp], _ = codec.write_kv(raw, zero, mini_slots, bits)
    bt = np.arange(npg, dtype=np.int32)[None]
    q = queries[b, h][None, None]
    return oracle.paged_decode_heads(q, pages["k"], pages["v"], bt, np.array([L]), w.k_bits, w.v_bits,
                                     codec.signs, codec.centroids32(w.k_bits), codec.centroids32(w.v_bits),
                                     [(0, 0)])[0]


def _samples(w, name):
    B, Hq = w.batch, w.num_q_heads
    if name == "ragged_write":
        order = np.argsort(w.seq_lens)
        bs = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
        return [(bs[0], 0), (bs[1], min(Hq - 1, Hq // 2 + 1)), (bs[2], Hq - 1)]
    if name == "long_context":  # 131072-token sequences: two samples keep the oracle under a minute
        return [(0, 0), (B - 1, Hq - 1)]
    return [(0, 0), (B // 2, min(Hq - 1, Hq // 2 + 1)), (B - 1, Hq - 1)]


@pytest.mark.parametrize("name", ["tiny", "pages_geometry", "mixed_bits", "long_context", "ragged_write"])
def test_full_size_sampled_outputs(ctx, name):
    w = workloads.preset(name)
    print(f"[fullsize] {name}: B={w.batch} Lmax={w.max_seq_len} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"K{w.k_bits}V{w.v_bits} tokens={w.num_tokens}", flush=True)
    out = _gpu_path(ctx, w)
    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    queries = w.queries()
    picks = _samples(w, name)
    got = np.stack([out[b, h] for b, h in picks])
    ref = np.stack([_oracle_head(w, codec, b, h, queries) for b, h in picks])
    r = compare_decode(got, ref, f"{name} sampled {picks}")
    print(f"  sampled {picks}: max|d| relL2 {r}", flush=True)
