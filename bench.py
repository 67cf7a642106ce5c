"""Benchmark of the TQ packed-page decode step on one MI355X.

A step is one decode step of the whole hot path for a batch of sequences:
write the new token's K row and V row of every sequence into the pages
(tq_write_kv, the row writer), then run the single-query paged decode over
each sequence's full context (tq_paged_decode).  The workload defaults to
the long-context configuration: 8 sequences x 131072 tokens, K4/V4, 64 query
heads over 8 KV heads, head_dim 128, 16-token pages in a random permutation
(1.14 GB of packed K+V).

Prints one JSON line (rank 0).  ``value`` is decode tokens/s (sequences x
steps / time); ``packed_kv_gbps`` is the packed K+V bytes of the context over
the decode time.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(w, kraw, vraw, q, seconds=15.0):
    """Time the oracle (as it stands) on one sequence, a subset of KV heads."""
    import oracle

    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    ck, cv = codec.centroids32(w.k_bits), codec.centroids32(w.v_bits)
    b = 0
    L = int(w.seq_lens[b])
    G = w.num_q_heads // w.num_kv_heads
    lo = int(w.cu_seqlens[b])
    t_total, groups = 0.0, 0
    t0 = time.perf_counter()
    for g in range(w.num_kv_heads):
        # encode this KV head's rows of sequence b (the oracle writer), then decode its query heads
        ts = time.perf_counter()
        krows, _ = codec.encode_bytes(kraw[lo:lo + L, g], w.k_bits)
        vrows, _ = codec.encode_bytes(vraw[lo:lo + L, g], w.v_bits)
        t_enc = time.perf_counter() - ts
        ts = time.perf_counter()
        K = codec.dequantize(krows, w.k_bits)
        V = codec.dequantize(vrows, w.v_bits)
        for h in range(g * G, (g + 1) * G):
            s = (K @ q[b, h].astype(np.float64)) / np.sqrt(w.head_dim)
            p = np.exp(s - s.max())
            _ = (p / p.sum()) @ V
        t_total += time.perf_counter() - ts
        groups += 1
        del t_enc
        if time.perf_counter() - t0 > seconds:
            break
    t_seq = t_total / groups * w.num_kv_heads  # decode of one whole sequence (all heads)
    bytes_seq = L * w.num_kv_heads * (w.row_bytes(w.k_bits) + w.row_bytes(w.v_bits))
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {
        "value": 1.0 / t_seq,
        "unit": "decode tokens/s",
        "packed_kv_gbps": bytes_seq / t_seq / 1e9,
        "cores": cores,
        "kind": "oracle",
        "sample": f"sequence 0 ({L} tokens), {groups} of {w.num_kv_heads} KV heads x {G} query heads, "
                  f"float64 dequantise-then-softmax, scaled to all heads",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="long_context")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_decode_attention_tq_amd import api, workloads

    dev = torch.device("cuda:0")
    w = workloads.preset(args.config)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    log(f"[bench] {w.name}: B={B} L={w.max_seq_len} Hq={Hq} Hkv={Hkv} K{w.k_bits}V{w.v_bits} "
        f"packed={w.packed_kv_bytes() / 1e9:.3f} GB")

    t0 = time.perf_counter()
    kraw, vraw, q = w.rows("k", threads=16), w.rows("v", threads=16), w.queries()
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f}s")
    ctx = api.Context(d, w.rht_seed)
    kp = torch.zeros(w.page_shape(w.k_bits), dtype=torch.uint8, device=dev)
    vp = torch.zeros(w.page_shape(w.v_bits), dtype=torch.uint8, device=dev)
    slots = torch.from_numpy(w.slots).to(dev)
    kraw_d = torch.from_numpy(kraw).to(dev)
    vraw_d = torch.from_numpy(vraw).to(dev)
    api.write_kv(ctx, kraw_d, kp, slots, w.k_bits)
    api.write_kv(ctx, vraw_d, vp, slots, w.v_bits)
    torch.cuda.synchronize()
    log("[bench] pages written (prefill)")

    # per-step inputs: the last token of every sequence is (re)written each step
    last = torch.from_numpy((w.cu_seqlens[1:] - 1).astype(np.int64)).to(dev)
    new_slots = slots[last].contiguous()
    k_new = kraw_d[last].contiguous()
    v_new = vraw_d[last].contiguous()
    q_d = torch.from_numpy(q).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws = torch.empty(api.decode_workspace_bytes(ctx, B, Hq, Hkv, w.max_seq_len), dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    del kraw_d, vraw_d

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(i=None):
        api.write_kv(ctx, k_new, kp, new_slots, w.k_bits, err_count=err, check_slots=False)
        api.write_kv(ctx, v_new, vp, new_slots, w.v_bits, err_count=err, check_slots=False)
        if i is not None:
            ev[i][0].record()
        api.paged_decode(ctx, q_d, kp, vp, bt, lens, w.k_bits, w.v_bits, max_seq_len=w.max_seq_len,
                         out=out, workspace=ws)
        if i is not None:
            ev[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert int(err.item()) == 0
    dec_ms = np.array([a.elapsed_time(b) for a, b in ev])
    log(f"[bench] decode ms per call: mean {dec_ms.mean():.4f} median {np.median(dec_ms):.4f} min {dec_ms.min():.4f}")

    ms_step = elapsed * 1e3 / args.steps
    packed = w.packed_kv_bytes()
    dec_s = float(dec_ms.mean()) / 1e3
    achieved = packed / dec_s / 1e9
    result = {
        "metric": "paged TQ decode tokens/s + packed-KV HBM GB/s (% of peak), 1 MI355X",
        "value": B / (ms_step / 1e3),
        "unit": "decode tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA operands (hi+lo split), fp32 accumulation; u8 packed K4/V4",
        "data": "synthetic (seeded N(0,1) fp16 K/V/q, random page permutation)",
        "config": {
            "workload": f"{w.name}: batch {B} x {w.max_seq_len} tokens, Hq {Hq}, Hkv {Hkv}, head_dim {d}, "
                        f"block 16, K{w.k_bits}/V{w.v_bits}",
            "global_batch": B,
            "seq_len": w.max_seq_len,
            "parallelism": "single GPU",
        },
        "packed_kv_bytes": packed,
        "decode_ms": float(dec_ms.mean()),
        "decode_ms_min": float(dec_ms.min()),
        "packed_kv_gbps": achieved,
        "pct_hbm_peak": 100.0 * achieved / HBM_PEAK_GBPS,
        "context_tokens_per_s": float(w.num_tokens) / dec_s,
        "roofline": {
            "bound": "hbm",
            "kernel": "tq_paged_decode (split + merge kernels)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": None,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        result["cpu_baseline"] = cpu_baseline(w, kraw, vraw, q, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
