"""GPU parity at the full workload sizes.

Every configuration runs at its full size through the GPU path in the
configuration the benchmark times: the row writer encodes every row of every
sequence into the pages (through the flat slots, with dropped slots where the
workload has them), then one decode over all sequences.  For two sampled
sequences per configuration (the only one for the tiny case; the shortest
and the longest of the ragged batch) the oracle then, from the same seeded
raw rows and nothing the GPU produced:

* encodes every row of the sequence, all KV heads, K and V, into its own
  pages, which must equal the GPU-written pages of that sequence byte for
  byte (gathered through its block table), up to the near-boundary
  exemption: a differing index must sit within 1e-6 of a codebook boundary
  and such indices must be fewer than 1e-4 of the sequence's indices; norm
  bytes have no exemption;
* decodes every query head of the sequence from its own pages; the GPU
  outputs of those heads must be within max-abs 2e-3 and relative L2 1e-3.

Margins (max |d|, relative L2, near-boundary mismatches) are printed, and
appended as JSON lines to the file named by TQ_PARITY_RECORD when it is set.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import api, workloads
from tests.oracle_par import sequence_outputs, sequence_pages
from tests.parity import compare_decode, compare_pages

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
    return out.cpu().numpy(), kp, vp


def _sampled_sequences(w, name):
    if w.batch == 1:
        return [0]
    if name == "ragged_write":
        order = np.argsort(w.seq_lens, kind="stable")
        return [int(order[0]), int(order[-1])]
    return [0, w.batch - 1]


def _record(entry):
    path = os.environ.get("TQ_PARITY_RECORD")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(entry) + "\n")


@pytest.mark.parametrize("name", ["tiny", "pages_geometry", "mixed_bits", "long_context", "ragged_write"])
def test_full_size_pages_and_outputs(ctx, name):
    w = workloads.preset(name)
    print(f"[fullsize] {name}: B={w.batch} Lmax={w.max_seq_len} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"K{w.k_bits}V{w.v_bits} tokens={w.num_tokens}", flush=True)
    out, kp, vp = _gpu_path(ctx, w)
    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    queries = w.queries()
    for b in _sampled_sequences(w, name):
        L = int(w.seq_lens[b])
        npg = (L + w.block_size - 1) // w.block_size
        ids = torch.from_numpy(w.block_table[b, :npg].astype(np.int64)).to(kp.device)
        ref_pages = {}
        entry = {"config": name, "sequence": b, "tokens": L}
        for comp, gpu_pages, bits in (("k", kp, w.k_bits), ("v", vp, w.v_bits)):
            pages, near, kept = sequence_pages(codec, w, b, comp, bits)
            got = gpu_pages[ids].cpu().numpy()
            n_bad, total = compare_pages(got, pages, near, bits, kept * w.num_kv_heads)
            entry[f"{comp}_near_mismatch"] = n_bad
            entry[f"{comp}_indices"] = total
            entry[f"{comp}_near_coords"] = int(near.sum())
            ref_pages[comp] = pages
            print(f"  seq {b} ({L} tokens) {comp.upper()} pages: near-boundary mismatches {n_bad}/{total}", flush=True)
        ref = sequence_outputs(codec, w, b, ref_pages["k"], ref_pages["v"], queries)
        max_abs, rel = compare_decode(out[b], ref, f"{name} sequence {b}, all {w.num_q_heads} heads")
        entry.update(max_abs=max_abs, rel_l2=rel, out_max=float(np.abs(ref).max()))
        print(f"  seq {b}: all heads max|d|={max_abs:.3e} relL2={rel:.3e} (max|out|={entry['out_max']:.3g})",
              flush=True)
        _record(entry)
