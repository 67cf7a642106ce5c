"""Benchmark of the TQ packed-page decode step on one MI355X.

A step is one decode step of the whole hot path for a batch of sequences:
write the new token's K row and V row of every sequence into the pages
(the row writer, K and V in one launch: tq_write_kv_pair), then run the single-query paged decode over
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
    """Time the oracle, as it stands, on a bounded sample of the workload.

    The sample is the first ``Ls`` tokens of sequence 0 (all KV heads): the
    oracle writer builds its pages, then ``oracle.paged_decode_heads`` decodes
    whole query groups until about ``seconds`` have been spent.  The decode
    time of one group is scaled to a full step (every group of every
    sequence, at the full context length).
    """
    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl is optional
        blas_threads = None
    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    L = int(w.seq_lens[0])
    Ls = min(L, 32768)
    G = w.num_q_heads // w.num_kv_heads
    lo = int(w.cu_seqlens[0])
    npg = (Ls + w.block_size - 1) // w.block_size
    bt = np.arange(npg, dtype=np.int32)[None]
    slots = np.arange(Ls, dtype=np.int64)
    kp = np.zeros((npg, w.block_size, w.num_kv_heads, w.row_bytes(w.k_bits)), dtype=np.uint8)
    vp = np.zeros((npg, w.block_size, w.num_kv_heads, w.row_bytes(w.v_bits)), dtype=np.uint8)
    t0 = time.perf_counter()
    kp, _ = codec.write_kv(kraw[lo:lo + Ls], kp, slots, w.k_bits)
    vp, _ = codec.write_kv(vraw[lo:lo + Ls], vp, slots, w.v_bits)
    t_write = time.perf_counter() - t0
    ck, cv = codec.centroids32(w.k_bits), codec.centroids32(w.v_bits)
    t_dec, groups = 0.0, 0
    for g in range(w.num_kv_heads):
        heads = [(0, h) for h in range(g * G, (g + 1) * G)]
        ts = time.perf_counter()
        oracle.paged_decode_heads(q[:1], kp, vp, bt, np.array([Ls]), w.k_bits, w.v_bits, codec.signs, ck, cv, heads)
        t_dec += time.perf_counter() - ts
        groups += 1
        if t_dec > seconds:
            break
    t_group = t_dec / groups
    t_step = t_group * w.num_kv_heads * w.batch * (L / Ls)  # every group of every sequence, full context
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {
        "value": w.batch / t_step,
        "unit": "decode tokens/s",
        "packed_kv_gbps": w.packed_kv_bytes() / t_step / 1e9,
        "write_rows_per_s": 2 * Ls * w.num_kv_heads / t_write,
        "cores": blas_threads if blas_threads else cores,
        "host_cores": cores,
        "kind": "oracle",
        "sample": f"sequence 0, first {Ls} of {L} tokens, {groups} of {w.num_kv_heads} KV-head groups x {G} query "
                  f"heads decoded by oracle.paged_decode_heads (float64) in {t_dec:.1f} s, scaled to "
                  f"{w.batch} sequences x {L} tokens x {w.num_kv_heads} groups; oracle write of the sample "
                  f"({Ls} tokens x {w.num_kv_heads} heads, K and V) took {t_write:.1f} s",
    }


def _oracle_sample(w, kraw, vraw, Ls):
    """The oracle writer's pages of the first ``Ls`` tokens of sequence 0 (all
    KV heads, identity block table) and the time the write took."""
    import oracle

    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    lo = int(w.cu_seqlens[0])
    npg = (Ls + w.block_size - 1) // w.block_size
    slots = np.arange(Ls, dtype=np.int64)
    kp = np.zeros((npg, w.block_size, w.num_kv_heads, w.row_bytes(w.k_bits)), dtype=np.uint8)
    vp = np.zeros((npg, w.block_size, w.num_kv_heads, w.row_bytes(w.v_bits)), dtype=np.uint8)
    t0 = time.perf_counter()
    kp, _ = codec.write_kv(kraw[lo:lo + Ls], kp, slots, w.k_bits)
    vp, _ = codec.write_kv(vraw[lo:lo + Ls], vp, slots, w.v_bits)
    return codec, kp, vp, np.arange(npg, dtype=np.int32)[None], time.perf_counter() - t0


def cpu_path_baseline(w, kraw, vraw, seconds, call, per_step, unit, what):
    """Time an oracle attention function on the first ``Ls`` tokens of
    sequence 0, one KV head (its pages' head slice and its query heads) per
    call, until about ``seconds`` have been spent; the time of one KV head is
    scaled to a full step (every KV head of every sequence, the full
    context).  ``call(codec, kp, vp, bt, Ls, g)`` runs the oracle for KV head
    g; ``per_step`` is the step's count in ``unit``."""
    L = int(w.seq_lens[0])
    Ls = min(L, 32768)
    codec, kp, vp, bt, t_write = _oracle_sample(w, kraw, vraw, Ls)
    t_run, heads = 0.0, 0
    for g in range(w.num_kv_heads):
        kg = np.ascontiguousarray(kp[:, :, g:g + 1])
        vg = np.ascontiguousarray(vp[:, :, g:g + 1])
        ts = time.perf_counter()
        call(codec, kg, vg, bt, Ls, g)
        t_run += time.perf_counter() - ts
        heads += 1
        if t_run > seconds:
            break
    t_step = t_run / heads * w.num_kv_heads * w.batch * (L / Ls)
    return {"value": per_step / t_step, "unit": unit, "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"sequence 0, first {Ls} of {L} tokens, {heads} of {w.num_kv_heads} KV heads by {what} "
                      f"(float64) in {t_run:.1f} s, scaled to {w.batch} sequences x {L} tokens x "
                      f"{w.num_kv_heads} KV heads; oracle write of the sample took {t_write:.1f} s"}


def op_traffic_bytes(op, key):
    """HBM bytes per call of an op on a workload from the committed counter
    profiles, if they were taken on the op's current sources (else None)."""
    import hashlib

    try:
        prof = json.load(open(os.path.join(ROOT, "profiles", "op_traffic.json")))
        rec = prof["ops"][op]
        digest = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])).hexdigest()
    except (OSError, ValueError, KeyError, TypeError):
        return None
    if rec.get("sources_sha256") != digest:
        return None
    return rec.get("bytes_per_call", {}).get(key)


def stream_read_ceiling(torch, dev, gib=2, reps=10):
    """Practical HBM read ceiling on this device: the streaming-read probe
    (csrc/probe/tq_stream_probe.hip, 16-byte non-temporal loads, 1 KB per wave
    instruction) over a ``gib`` GiB buffer, timed with events; GB/s (best, mean)."""
    import ctypes

    path = os.path.join(ROOT, "paged_decode_attention_tq_amd", "libtq_probe.so")
    lib = ctypes.CDLL(path)
    lib.tq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p]
    lib.tq_probe_stream_read.restype = ctypes.c_int
    nbytes = gib << 30
    blocks = 2048
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(blocks * 512, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def run():
        st = lib.tq_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, stream)
        if st != 0:
            raise RuntimeError(f"stream-read probe launch failed (hip error {st})")

    for _ in range(3):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    del buf, sink
    return {"kernel": "tq_probe_stream_read (16-byte non-temporal loads)", "bytes": nbytes,
            "best_gbps": nbytes / (ms.min() / 1e3) / 1e9, "mean_gbps": nbytes / (ms.mean() / 1e3) / 1e9}


def traffic_bytes(config):
    """HBM bytes per decode call of this config from the committed counter
    profile, if it was taken on the current decode sources (else None)."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    try:
        prof = json.load(open(path))
        digest = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in prof["sources"])).hexdigest()
    except (OSError, ValueError, KeyError, TypeError):
        return None
    if prof.get("decode_sources_sha256") != digest:
        return None
    return prof.get("configs", {}).get(config, {}).get("bytes_per_call")


def prod_traffic_bytes(config):
    """HBM bytes per tq_prod_scores call of this config from the committed
    counter profile, if it was taken on the current prod sources (else None)."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "prod_traffic.json")
    try:
        prof = json.load(open(path))
        digest = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in prof["sources"])).hexdigest()
    except (OSError, ValueError, KeyError, TypeError):
        return None
    if prof.get("prod_sources_sha256") != digest:
        return None
    return prof.get("configs", {}).get(config, {}).get("scores_bytes_per_call")


def cpu_decompress_baseline(w, kp_host, seconds=15.0):
    """Time the oracle's readback (``oracle.decompress_kv``) on a bounded
    sample: blocks of 2048 tokens (all KV heads) of the workload's slots,
    repeated until about ``seconds`` have been spent; rows/s."""
    import oracle

    codec = oracle.OracleCodec(w.head_dim, w.rht_seed)
    rows, t0 = 0, time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        s = w.slots[i * 2048:(i + 1) * 2048]
        codec.decompress_kv(kp_host, s, w.k_bits)
        rows += len(s) * w.num_kv_heads
        i += 1
    el = time.perf_counter() - t0
    return {"value": rows / el, "unit": "rows/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{i} blocks of 2048 tokens x {w.num_kv_heads} KV heads of the workload's K pages, {el:.1f} s"}


def bench_decompress(args, torch, api, w, ctx, kp, slots):
    """Dense readback of every K row of the workload (one tq_decompress_kv call
    over all tokens), timed with events on the library's stream."""
    dt = {"fp16": torch.float16, "bf16": torch.bfloat16, "fp32": torch.float32}[args.out_dtype]
    dev = kp.device
    N, Hkv, d = w.num_tokens, w.num_kv_heads, w.head_dim
    out = torch.empty((N, Hkv, d), dtype=dt, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush_rd = None if args.no_flush else torch.ones(1 << 27, dtype=torch.int64, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def call(i=None):
        if flush is not None:
            flush.zero_()
            flush_rd.sum()
        if i is not None:
            ev[i][0].record()
        api.decompress_kv(ctx, kp, slots, w.k_bits, out=out, err_count=err, check_slots=False)
        if i is not None:
            ev[i][1].record()

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    rows = N * Hkv
    kept = int((w.slots >= 0).sum()) * Hkv
    nbytes = 8 * N + kept * w.row_bytes(w.k_bits) + rows * d * out.element_size()
    sec = float(ms.mean()) / 1e3
    log(f"[bench] decompress ms per call: mean {ms.mean():.4f} median {np.median(ms):.4f} min {ms.min():.4f}")
    result = {
        "metric": "TQ dense readback rows/s + HBM GB/s (% of peak), 1 MI355X",
        "value": rows / sec,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": float(ms.mean()),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"u8 packed K{w.k_bits} rows in, fp32 reconstruction, {args.out_dtype} rows out",
        "data": "synthetic (the workload's K rows written by the row writer)",
        "config": {"workload": f"{w.name} K pages: {N} tokens x Hkv {Hkv}, head_dim {d}, block 16, K{w.k_bits}, "
                               f"{args.out_dtype} out", "rows": rows},
        "decompress_ms": float(ms.mean()),
        "decompress_ms_median": float(np.median(ms)),
        "decompress_ms_min": float(ms.min()),
        "roofline": {
            "bound": "hbm",
            "kernel": "tq_decompress_kv (decompress_rows_kernel)",
            "achieved": nbytes / sec / 1e9,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": nbytes / sec / 1e9 / HBM_PEAK_GBPS,
            "algorithmic_bytes": nbytes,
            "traffic": op_traffic_bytes("decompress", f"{w.name}/{args.out_dtype}"),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle readback on the host")
        result["cpu_baseline"] = cpu_decompress_baseline(w, kp.cpu().numpy(), min(args.cpu_seconds, 15.0))
    return result


def cpu_prod_baseline(w, q, S, bits, seconds=15.0):
    """Time the oracle's estimator (``oracle.prod_scores``) on a bounded
    sample: the first 2048 tokens of sequence 0, written as prod rows by the
    oracle (untimed), scored against each KV head's query group in turn until
    about ``seconds`` have been spent; scores/s."""
    import oracle

    signs = oracle.rht_signs(w.rht_seed, w.head_dim)
    raw = w.seq_rows("k", 0)[:2048]
    T, Hkv = raw.shape[0], w.num_kv_heads
    RB = oracle.prod_row_bytes(w.head_dim, bits)
    pages = np.zeros(((T + 15) // 16, 16, Hkv, RB), dtype=np.uint8)
    pages, _, _ = oracle.write_prod(raw, pages, np.arange(T, dtype=np.int64), bits, signs, S)
    rows = pages.reshape(-1, Hkv, RB)[:T]
    G = w.num_q_heads // Hkv
    n, i, t0 = 0, 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        g = i % Hkv
        oracle.prod_scores(q[0, g * G:(g + 1) * G], rows[:, g], bits, signs, S)
        n += G * T
        i += 1
    el = time.perf_counter() - t0
    return {"value": n / el, "unit": "scores/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{i} calls of {T} tokens x {G} query heads (sequence 0, one KV head each), {el:.1f} s"}


def bench_prod(args, torch, api, w, ctx, kraw_d, slots, q):
    """The prod key codec on the workload's K rows: the writer over every row,
    then the inner-product scores of every query head over every key, timed
    with events (each after the cache flush)."""
    from paged_decode_attention_tq_amd import workloads

    dev = kraw_d.device
    bits = w.k_bits
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    RB = api.prod_row_bytes(d, bits)
    pages = torch.zeros((w.num_blocks, 16, Hkv, RB), dtype=torch.uint8, device=dev)
    S = torch.from_numpy(workloads.qjl_matrix(d, seed=0)).to(dev)
    q_d = torch.from_numpy(q).to(dev)
    bt, lens = torch.from_numpy(w.block_table).to(dev), torch.from_numpy(w.seq_lens).to(dev)
    scores = torch.empty((B, Hq, w.max_seq_len), dtype=torch.float32, device=dev)
    ws = torch.empty(2 * B * Hq * d * 4, dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush_rd = None if args.no_flush else torch.ones(1 << 27, dtype=torch.int64, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def call(i=None):
        for k, fn in enumerate((
                lambda: api.write_kv_prod(ctx, kraw_d, pages, slots, bits, S, err_count=err, check_slots=False),
                lambda: api.prod_scores(ctx, q_d, pages, bt, lens, bits, S, max_seq_len=w.max_seq_len, out=scores,
                                        workspace=ws))):
            if flush is not None:
                flush.zero_()
                flush_rd.sum()
            if i is not None:
                ev[i][2 * k].record()
            fn()
            if i is not None:
                ev[i][2 * k + 1].record()

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    wms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    sms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    rows = kraw_d.shape[0] * Hkv
    kept = int((w.slots >= 0).sum()) * Hkv
    wbytes = kraw_d.numel() * kraw_d.element_size() + kept * RB
    sbytes = w.num_tokens * Hkv * RB + B * Hq * w.max_seq_len * 4
    log(f"[bench] prod writer ms: mean {wms.mean():.4f}; scores ms: mean {sms.mean():.4f}")
    ssec = float(sms.mean()) / 1e3
    return {
        "metric": "TQ prod key codec: scores (key-query inner products)/s + HBM GB/s (% of peak), 1 MI355X",
        "value": Hq * w.num_tokens / ssec,
        "unit": "scores/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": float(sms.mean()),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"u8 prod rows ({bits - 1}-bit indices + 1-bit sketch); fp16 hi+lo MFMA operands, fp32 accumulation",
        "data": "synthetic (the workload's K rows; a seeded Gaussian sketch matrix)",
        "config": {"workload": f"{w.name} K rows as {bits}-bit prod rows: {w.num_tokens} tokens x Hkv {Hkv}, "
                               f"Hq {Hq}, head_dim {d}, block 16"},
        "scores_ms": float(sms.mean()), "scores_ms_min": float(sms.min()),
        "writer_ms": float(wms.mean()), "writer_rows_per_s": rows / (float(wms.mean()) / 1e3),
        "writer_gbps": wbytes / (float(wms.mean()) / 1e3) / 1e9,
        "roofline": {"bound": "hbm", "kernel": "tq_prod_scores (prod_query_kernel + prod_scores_kernel)",
                     "achieved": sbytes / ssec / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": sbytes / ssec / 1e9 / HBM_PEAK_GBPS, "algorithmic_bytes": sbytes,
                     "traffic": prod_traffic_bytes(w.name)},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_prod_baseline(
            w, q, workloads.qjl_matrix(d, seed=0), bits, min(args.cpu_seconds, 15.0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="long_context")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ceiling", action="store_true", help="skip the streaming-read ceiling probe")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-flush", action="store_true", help="skip the cache flush (1 GiB write, then 1 GiB read) before each timed step")
    ap.add_argument("--op", choices=("decode", "append", "decompress", "hybrid", "prefill", "prod"), default="decode",
                    help="decode: the decode step (default); append: the same step as one call that writes the new "
                         "rows inside the decode (tq_paged_decode_append); decompress: the dense readback of every K row; "
                         "hybrid: the decode step over the packed pages plus an exact fp16 window per sequence; "
                         "prefill: a chunk of --q-len queries per sequence attending causally over the pages; "
                         "prod: the prod key codec (writer of every K row, then every head's scores over them)")
    ap.add_argument("--q-len", type=int, default=8, help="queries per sequence (--op prefill)")
    ap.add_argument("--window", type=int, default=128, help="recent-window rows per sequence (--op hybrid)")
    ap.add_argument("--out-dtype", choices=("fp16", "bf16", "fp32"), default="fp16",
                    help="output dtype of the dense readback (--op decompress)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_decode_attention_tq_amd import api, workloads

    dev = torch.device("cuda:0")
    w = workloads.preset(args.config)
    kernel = api.decode_kernel(w.batch, w.num_q_heads * (args.q_len if args.op == "prefill" else 1), w.num_kv_heads,
                               w.max_seq_len, w.k_bits, w.v_bits)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    log(f"[bench] {w.name}: B={B} L={w.max_seq_len} Hq={Hq} Hkv={Hkv} K{w.k_bits}V{w.v_bits} "
        f"packed={w.packed_kv_bytes() / 1e9:.3f} GB, {kernel} decode kernel")

    t0 = time.perf_counter()
    kraw, vraw, q = w.rows("k", threads=16), w.rows("v", threads=16), w.queries()
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f}s")
    ctx = api.Context(d, w.rht_seed)
    kp = torch.zeros(w.page_shape(w.k_bits), dtype=torch.uint8, device=dev)
    vp = torch.zeros(w.page_shape(w.v_bits), dtype=torch.uint8, device=dev)
    slots = torch.from_numpy(w.slots).to(dev)
    kraw_d = torch.from_numpy(kraw).to(dev)
    vraw_d = torch.from_numpy(vraw).to(dev)
    # the prefill (every row of every sequence, K then V), timed as the row
    # writer's throughput: raw rows read + packed rows written
    warm_slot = torch.zeros(1, dtype=torch.int64, device=dev)  # first launches of both writers, on a spare page
    for pages_shape, bits, raw in ((w.page_shape(w.k_bits), w.k_bits, kraw_d), (w.page_shape(w.v_bits), w.v_bits, vraw_d)):
        spare = torch.zeros((1,) + tuple(pages_shape[1:]), dtype=torch.uint8, device=dev)
        api.write_kv(ctx, raw[:1].contiguous(), spare, warm_slot, bits)
    torch.cuda.synchronize()
    wev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    wev[0].record()
    api.write_kv(ctx, kraw_d, kp, slots, w.k_bits)
    wev[1].record()
    api.write_kv(ctx, vraw_d, vp, slots, w.v_bits)
    wev[2].record()
    torch.cuda.synchronize()
    write_s = wev[0].elapsed_time(wev[2]) / 1e3
    kept = int((w.slots >= 0).sum()) * Hkv
    write_bytes = kraw_d.numel() * kraw_d.element_size() + vraw_d.numel() * vraw_d.element_size() + \
        kept * (w.row_bytes(w.k_bits) + w.row_bytes(w.v_bits))
    write = {"rows": 2 * kraw_d.shape[0] * Hkv, "ms": write_s * 1e3, "rows_per_s": 2 * kraw_d.shape[0] * Hkv / write_s,
             "gbps": write_bytes / write_s / 1e9, "bytes": write_bytes}
    log(f"[bench] pages written (prefill): {write['rows']} rows in {write['ms']:.3f} ms, "
        f"{write['rows_per_s'] / 1e6:.1f} M rows/s, {write['gbps']:.0f} GB/s")

    if args.op == "prod":
        del vraw_d
        print(json.dumps(bench_prod(args, torch, api, w, ctx, kraw_d, slots, q)), flush=True)
        return
    if args.op == "decompress":
        del kraw_d, vraw_d
        print(json.dumps(bench_decompress(args, torch, api, w, ctx, kp, slots)), flush=True)
        return

    # per-step inputs: the last token of every sequence is (re)written each step
    last = torch.from_numpy((w.cu_seqlens[1:] - 1).astype(np.int64)).to(dev)
    new_slots = slots[last].contiguous()
    k_new = kraw_d[last].contiguous()
    v_new = vraw_d[last].contiguous()
    q_d = torch.from_numpy(q).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    hybrid = args.op == "hybrid"
    prefill = args.op == "prefill"
    append = args.op == "append"
    if prefill:
        # the last q_len tokens of every sequence query the pages (their rows are
        # rewritten each step like the decode step's new token)
        Lq = args.q_len
        pq = torch.from_numpy(np.random.default_rng(5).standard_normal((B, Lq, Hq, d), dtype=np.float32)).to(
            device=dev, dtype=torch.float16)
        ql_d = torch.full((B,), Lq, dtype=torch.int32, device=dev)
        out = torch.empty((B, Lq, Hq, d), dtype=torch.float32, device=dev)
        ws = torch.empty(api.prefill_workspace_bytes(ctx, B, Lq, Hq, Hkv, w.max_seq_len), dtype=torch.uint8,
                         device=dev)
    elif hybrid:
        # a full window of exact rows per sequence, fp16, drawn like the workload's rows
        rl = np.full(B, args.window, dtype=np.int32)
        rk, rv = w.recent_window(args.window, rl, seed=1)
        rk_d, rv_d = torch.from_numpy(rk).to(dev), torch.from_numpy(rv).to(dev)
        rl_d = torch.from_numpy(rl).to(dev)
        ws = torch.empty(api.hybrid_workspace_bytes(ctx, B, Hq, Hkv, w.max_seq_len), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(api.decode_workspace_bytes(ctx, B, Hq, Hkv, w.max_seq_len), dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    del kraw_d, vraw_d

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    # Before each timed step, untimed: write 1 GiB (evicts the pages from L2
    # and the 256 MB MALL), then read another 1 GiB.  The read pass makes the
    # caches write back the memset's dirty lines before the timed region;
    # without it that write-back (up to the MALL's 256 MB) lands inside the
    # decode and is charged to it.
    flush = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush_rd = None if args.no_flush else torch.ones(1 << 27, dtype=torch.int64, device=dev)

    def step(i=None):
        # timed: the row writer for the new token of every sequence, then the decode
        if flush is not None:
            flush.zero_()
            flush_rd.sum()
        if i is not None:
            ev[i][0].record()
        if not append:
            api.write_kv_pair(ctx, k_new, v_new, kp, vp, new_slots, w.k_bits, w.v_bits, err_count=err,
                              check_slots=False)
        if i is not None:
            ev[i][1].record()
        if append:  # the new rows are written by the decode kernel itself
            api.paged_decode_append(ctx, q_d, k_new, v_new, kp, vp, bt, lens, w.k_bits, w.v_bits,
                                    max_seq_len=w.max_seq_len, out=out, workspace=ws, err_count=err,
                                    check_pages=False)
        elif prefill:
            api.paged_prefill(ctx, pq, ql_d, kp, vp, bt, lens, w.k_bits, w.v_bits, max_seq_len=w.max_seq_len,
                              out=out, workspace=ws)
        elif hybrid:
            api.paged_decode_hybrid(ctx, q_d, kp, vp, bt, lens, rk_d, rv_d, rl_d, w.k_bits, w.v_bits,
                                    max_seq_len=w.max_seq_len, out=out, workspace=ws)
        else:
            api.paged_decode(ctx, q_d, kp, vp, bt, lens, w.k_bits, w.v_bits, max_seq_len=w.max_seq_len,
                             out=out, workspace=ws)
        if i is not None:
            ev[i][2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert int(err.item()) == 0
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    step_ms = np.array([e[0].elapsed_time(e[2]) for e in ev])
    log(f"[bench] decode ms per call: mean {dec_ms.mean():.4f} median {np.median(dec_ms):.4f} min {dec_ms.min():.4f}")

    ms_step = float(step_ms.mean())
    log(f"[bench] step (write + decode) ms: mean {ms_step:.4f}; wall per step incl. cache flush "
        f"{elapsed * 1e3 / args.steps:.4f}")
    packed = w.packed_kv_bytes()
    window_bytes = 0
    if hybrid:  # the window rows read (K and V, fp16) count as algorithmic bytes too
        window_bytes = 2 * B * args.window * Hkv * d * 2
        packed += window_bytes
    dec_s = float(dec_ms.mean()) / 1e3
    achieved = packed / dec_s / 1e9
    result = {
        "metric": ("paged TQ decode tokens/s + packed-KV HBM GB/s (% of peak), 1 MI355X" if not (hybrid or prefill
                                                                                            or append)
                   else "paged TQ decode step as one call (new rows written by the decode) tokens/s + packed-KV HBM "
                   "GB/s (% of peak), 1 MI355X" if append else f"paged TQ hybrid decode (packed history + {args.window}-row exact fp16 window) tokens/s + "
                   "HBM GB/s (% of peak), 1 MI355X" if hybrid else
                   f"paged TQ multi-query attention ({args.q_len} causal queries per sequence) query tokens/s + "
                   "packed-KV HBM GB/s (% of peak), 1 MI355X"),
        "value": B * (args.q_len if prefill else 1) / (ms_step / 1e3),
        "unit": "decode tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"u8 packed K{w.k_bits}/V{w.v_bits} pages; keys, queries and softmax weights as fp16 hi+lo MFMA "
                  "operands, value centroids fp16 (hi only, pre-scaled), fp32 accumulation"),
        "data": "synthetic (seeded N(0,1) fp16 K/V/q, random page permutation)",
        "config": {
            "workload": f"{w.name}: batch {B} x {w.max_seq_len} tokens, Hq {Hq}, Hkv {Hkv}, head_dim {d}, "
                        f"block 16, K{w.k_bits}/V{w.v_bits}" +
                        (f", plus a {args.window}-row fp16 window per sequence" if hybrid else "") +
                        (f", {args.q_len} fp16 queries per sequence" if prefill else ""),
            "global_batch": B,
            "seq_len": w.max_seq_len,
            "parallelism": "single GPU",
        },
        "packed_kv_bytes": packed,
        "decode_ms": float(dec_ms.mean()),
        "decode_ms_median": float(np.median(dec_ms)),
        "decode_ms_min": float(dec_ms.min()),
        "packed_kv_gbps": achieved,
        "pct_hbm_peak": 100.0 * achieved / HBM_PEAK_GBPS,
        "context_tokens_per_s": float(w.num_tokens) / dec_s,
        "roofline": {
            "bound": "hbm",
            "kernel": (("tq_paged_decode_append" if append else "tq_paged_decode") +
                       (f", {kernel} decode kernel + merge kernel" if kernel != "wave1" else
                        ", wave decode kernel as one workgroup (no merge kernel)") +
                       (" (the new rows encoded inside the decode kernel)" if append else "") +
                       (" + hybrid_window_kernel" if hybrid else "") +
                       (" + layout, tail readback and causal window kernels" if prefill else "")),
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": (op_traffic_bytes("hybrid", f"{w.name}/window{args.window}") if hybrid else
                        op_traffic_bytes("prefill", f"{w.name}/q{args.q_len}") if prefill else
                        op_traffic_bytes("append", w.name) if append else traffic_bytes(w.name)),
        },
        "prefill_write": write,
        "stream_read_ceiling": None,
        "cpu_baseline": None,
    }
    if not args.no_stream_ceiling:
        result["stream_read_ceiling"] = stream_read_ceiling(torch, dev)
        log(f"[bench] streaming-read ceiling: {result['stream_read_ceiling']['best_gbps']:.0f} GB/s best, "
            f"{result['stream_read_ceiling']['mean_gbps']:.0f} GB/s mean")
    if hybrid:
        result["window_bytes"] = window_bytes
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        if hybrid:
            import oracle

            rkh, rvh, rlh = rk[:1], rv[:1], rl[:1]
            G = Hq // Hkv

            def hyb(codec, kg, vg, bt, Ls, g):
                oracle.paged_decode_hybrid(q[:1, g * G:(g + 1) * G], kg, vg, bt, np.array([Ls]),
                                           rkh[:, :, g:g + 1], rvh[:, :, g:g + 1], rlh, w.k_bits, w.v_bits,
                                           codec.signs, codec.centroids32(w.k_bits), codec.centroids32(w.v_bits))

            result["cpu_baseline"] = cpu_path_baseline(w, kraw, vraw, args.cpu_seconds, hyb, B, "decode tokens/s",
                                                       "oracle.paged_decode_hybrid with the sequence's window")
        elif prefill:
            import oracle

            pqh = pq[:1].float().cpu().numpy()
            G = Hq // Hkv

            def pre(codec, kg, vg, bt, Ls, g):
                oracle.paged_prefill(pqh[:, :, g * G:(g + 1) * G], np.array([Lq]), kg, vg, bt, np.array([Ls]),
                                     w.k_bits, w.v_bits, codec.signs, codec.centroids32(w.k_bits),
                                     codec.centroids32(w.v_bits))

            result["cpu_baseline"] = cpu_path_baseline(w, kraw, vraw, args.cpu_seconds, pre, B * Lq,
                                                       "query tokens/s", f"oracle.paged_prefill ({Lq} queries)")
        else:
            result["cpu_baseline"] = cpu_baseline(w, kraw, vraw, q, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
