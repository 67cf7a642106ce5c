"""GPU parity of the prod key codec (tq_write_kv_prod) and its inner-product
scores (tq_prod_scores) against the oracle.

Writer: every stored row compared field by field with the oracle's encoding
of the same raw rows under the same sketch matrix: indices equal except at
near-boundary coordinates (as the MSE rows, and such rows are fewer than
1e-4 of all indices), norm bytes equal; on rows whose indices all match, the
sign bits equal except where the projection lies within fp32 rounding of
zero (marked by the oracle), and gamma (fp32 arithmetic on the GPU) within
2e-6 relative.

Scores: the GPU's estimate against the oracle's estimator over the same
page bytes, |d| <= 1e-5 * (|ref| + n * ||q||) per score (sums of 128
products in fp32); rel-L2 printed.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_tq_amd import api, workloads
from tests.oracle_par import sequence_prod_pages

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    return api.Context(128, 42)


def _compare_rows(got, ref, near_i, near_s, bits, what, check_fraction=True):
    """got / ref: prod row bytes [..., RB]; near masks [..., d].  Returns counts.
    check_fraction: mismatching indices under 1e-4 of all (rows drawn from the
    workloads' distributions; structured rows put coordinates on boundaries)."""
    d = 128
    gi, gn, gz, gg = oracle.prod_bytes_to_rows(got, bits, d)
    ri, rn, rz, rg = oracle.prod_bytes_to_rows(ref, bits, d)
    assert np.array_equal(gn.view(np.uint32), rn.view(np.uint32)), f"{what}: norm bytes differ"
    bad_i = gi != ri
    assert not (bad_i & ~near_i).any(), f"{what}: index mismatch away from a boundary"
    frac = bad_i.sum() / max(1, bad_i.size)
    assert frac < 1e-4 or not check_fraction, f"{what}: {bad_i.sum()} near-boundary index mismatches ({frac:.2e})"
    same = ~bad_i.any(axis=-1)
    bad_z = (gz != rz) & same[..., None]
    assert not (bad_z & ~near_s).any(), f"{what}: sign mismatch away from zero"
    np.testing.assert_allclose(gg[same], rg[same], rtol=2e-6, atol=1e-9, err_msg=f"{what}: gamma")
    print(f"  {what}: {int(bad_i.sum())} near-boundary index, {int(bad_z.sum())} near-zero sign mismatches "
          f"over {bad_i.size} coordinates", flush=True)


def _check_scores(got, ref, q, norms, what):
    tol = 1e-5 * (np.abs(ref) + norms * np.linalg.norm(q.astype(np.float64), axis=-1)[..., None])
    d = np.abs(got.astype(np.float64) - ref)
    assert (d <= tol).all(), f"{what}: worst excess {float((d - tol).max()):.3e}"
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    print(f"  {what}: max|d| {d.max():.3e} relL2 {rel:.3e}", flush=True)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_writer_matches_oracle(ctx, bits, dt):
    w = workloads.make_workload(f"qjl{bits}", num_q_heads=8, num_kv_heads=2, seq_lens=[300, 45, 129],
                                seed=110 + bits, drop_frac=0.1, lognormal_sigma=0.5, dtype=dt)
    print(f"[qjl] writer bits={bits} dtype={np.dtype(dt).name} N={w.num_tokens}", flush=True)
    S = workloads.qjl_matrix(128, seed=bits)
    signs = oracle.rht_signs(42, 128)
    shape = (w.num_blocks, 16, 2, oracle.prod_row_bytes(128, bits))
    ref, near_i, near_s = oracle.write_prod(w.rows("k"), np.zeros(shape, np.uint8), w.slots, bits, signs, S)
    pg = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    api.write_kv_prod(ctx, torch.from_numpy(w.rows("k")).cuda(), pg, torch.from_numpy(w.slots).cuda(), bits,
                      torch.from_numpy(S).cuda())
    torch.cuda.synchronize()
    got = pg.cpu().numpy()
    keep = w.slots[w.slots >= 0]
    _compare_rows(got[keep // 16, keep % 16], ref[keep // 16, keep % 16], near_i[keep // 16, keep % 16],
                  near_s[keep // 16, keep % 16], bits, f"bits {bits}")
    dropped_pages = np.ones(w.num_blocks * 16, bool)
    dropped_pages[keep] = False
    assert not got.reshape(w.num_blocks * 16, -1)[dropped_pages].any()  # skipped slots stay zero


# lengths past 512 tokens span several 32-page chunks of the score kernel;
# groups above 8 split a KV head's query heads over workgroups (12: a short tail);
# 601 columns take the scalar score stores; 8 and 16 KV heads put four
# neighbouring heads in one workgroup (one per wave)
@pytest.mark.parametrize("bits,hkv,G,lens", [(4, 2, 8, [200, 17, 0, 64]), (3, 1, 4, [200, 17, 0, 64]),
                                             (2, 4, 2, [200, 17, 0, 64]), (5, 2, 3, [200, 17, 0, 64]),
                                             (4, 1, 12, [1100, 17, 0, 530]), (3, 2, 16, [601, 513, 1]),
                                             (4, 8, 8, [1100, 17, 0, 530]), (3, 16, 2, [601, 45, 1])])
def test_scores_match_oracle(ctx, bits, hkv, G, lens):
    w = workloads.make_workload(f"qjls{bits}", num_q_heads=hkv * G, num_kv_heads=hkv, seq_lens=lens,
                                seed=120 + bits, outlier_frac=0.02)
    print(f"[qjl] scores bits={bits} Hkv={hkv} G={G} lens={w.seq_lens.tolist()}", flush=True)
    S = workloads.qjl_matrix(128, seed=20 + bits)
    signs = oracle.rht_signs(42, 128)
    shape = (w.num_blocks, 16, hkv, oracle.prod_row_bytes(128, bits))
    pages, _, _ = oracle.write_prod(w.rows("k"), np.zeros(shape, np.uint8), w.slots, bits, signs, S)
    q = w.queries()
    ref = oracle.paged_prod_scores(q, pages, w.block_table, w.seq_lens, bits, signs, S)
    got = api.prod_scores(ctx, torch.from_numpy(q).cuda(), torch.from_numpy(pages).cuda(),
                          torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(), bits,
                          torch.from_numpy(S).cuda())
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    norms = np.zeros(ref.shape)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        assert not got[b, :, L:].any()
        if L == 0:
            continue
        t = np.arange(L)
        rows = pages[w.block_table[b, t // 16], t % 16]  # [L, Hkv, RB]
        n = oracle.prod_bytes_to_rows(rows, bits, 128)[1].astype(np.float64)  # [L, Hkv]
        norms[b, :, :L] = np.repeat(n.T, G, axis=0)
    _check_scores(got, ref, q, norms, f"scores bits {bits}")


def test_full_size_long_context(ctx):
    # every K row of the long-context workload written as 4-bit prod rows on
    # the GPU, then the scores of every head over all 131072 tokens of each
    # sequence; sequence 0 checked row by row and score by score
    w = workloads.preset("long_context")
    bits = 4
    print(f"[qjl] full size long_context: {w.num_tokens} tokens x {w.num_kv_heads} heads, prod {bits} bits",
          flush=True)
    S = workloads.qjl_matrix(128, seed=4)
    signs = oracle.rht_signs(42, 128)
    dev = torch.device("cuda")
    pg = torch.zeros((w.num_blocks, 16, w.num_kv_heads, oracle.prod_row_bytes(128, bits)), dtype=torch.uint8,
                     device=dev)
    St = torch.from_numpy(S).to(dev)
    api.write_kv_prod(ctx, torch.from_numpy(w.rows("k", threads=16)).to(dev), pg, torch.from_numpy(w.slots).to(dev),
                      bits, St)
    q = w.queries()
    got = api.prod_scores(ctx, torch.from_numpy(q).to(dev), pg, torch.from_numpy(w.block_table).to(dev),
                          torch.from_numpy(w.seq_lens).to(dev), bits, St, max_seq_len=w.max_seq_len)
    torch.cuda.synchronize()
    b = 0
    L = int(w.seq_lens[b])
    ref_pages, near_i, near_s, kept = sequence_prod_pages(w, b, bits, signs, S)
    ids = torch.from_numpy(w.block_table[b, :L // 16].astype(np.int64)).to(dev)
    gpu_pages = pg[ids].cpu().numpy()
    _compare_rows(gpu_pages, ref_pages, near_i, near_s, bits, "long_context sequence 0")
    bt = np.arange(ref_pages.shape[0], dtype=np.int32)[None]
    ref = oracle.paged_prod_scores(q[b:b + 1], ref_pages, bt, np.array([L]), bits, signs, S)[0]
    # rows whose indices or signs differ (the exemptions above) are excluded;
    # gamma's last-place differences stay in (far inside the tolerance)
    gi, _, gz, _ = oracle.prod_bytes_to_rows(gpu_pages.reshape(L, w.num_kv_heads, -1), bits, 128)
    ri, _, rz, _ = oracle.prod_bytes_to_rows(ref_pages.reshape(L, w.num_kv_heads, -1), bits, 128)
    same = np.all(gi == ri, axis=-1) & np.all(gz == rz, axis=-1)
    G = w.num_q_heads // w.num_kv_heads
    mask = np.repeat(same.T, G, axis=0)  # [Hq, L]
    g = got[b].cpu().numpy()
    n = oracle.prod_bytes_to_rows(ref_pages.reshape(L, w.num_kv_heads, -1), bits, 128)[1].astype(np.float64)
    norms = np.repeat(n.T, G, axis=0)
    print(f"  {int((~mask).sum())} of {mask.size} scores excluded (rows with exempt index mismatches)", flush=True)
    _check_scores(np.where(mask, g, 0.0), np.where(mask, ref, 0.0), q[b], norms, "long_context sequence 0 scores")


def test_scores_bad_block_ids_read_zero_rows(ctx):
    # block ids outside [0, num_blocks) in the table read as zero rows: those
    # tokens score 0, every other token keeps the oracle's estimate
    bits = 4
    w = workloads.make_workload("qjlbad", num_q_heads=8, num_kv_heads=2, seq_lens=[300, 90], seed=131)
    S = workloads.qjl_matrix(128, seed=9)
    signs = oracle.rht_signs(42, 128)
    shape = (w.num_blocks, 16, 2, oracle.prod_row_bytes(128, bits))
    pages, _, _ = oracle.write_prod(w.rows("k"), np.zeros(shape, np.uint8), w.slots, bits, signs, S)
    q = w.queries()
    ref = oracle.paged_prod_scores(q, pages, w.block_table, w.seq_lens, bits, signs, S)
    bt = w.block_table.copy()
    bt[0, 3] = -1
    bt[0, 7] = w.num_blocks
    bt[1, 0] = w.num_blocks + 100
    print(f"[qjl] bad block ids: table entries (0,3) -1, (0,7) {w.num_blocks}, (1,0) {w.num_blocks + 100}", flush=True)
    got = api.prod_scores(ctx, torch.from_numpy(q).cuda(), torch.from_numpy(pages).cuda(),
                          torch.from_numpy(bt).cuda(), torch.from_numpy(w.seq_lens).cuda(), bits,
                          torch.from_numpy(S).cuda()).cpu().numpy()
    want = ref.copy()
    for b, p in ((0, 3), (0, 7), (1, 0)):
        want[b, :, 16 * p:16 * (p + 1)] = 0.0
    tol = 1e-5 * (np.abs(want) + 100.0)
    assert (np.abs(got - want) <= tol).all()
    assert not got[0, :, 48:64].any() and not got[0, :, 112:128].any() and not got[1, :, 0:16].any()


def test_writer_out_of_range_slots_are_counted_and_skipped(ctx):
    # slots past the pages raise the error count and write nothing (the
    # guard page behind the pages stays as it was)
    bits = 3
    w = workloads.make_workload("qjlslots", num_q_heads=4, num_kv_heads=2, seq_lens=[40], seed=132)
    S = torch.from_numpy(workloads.qjl_matrix(128, seed=2)).cuda()
    RB = oracle.prod_row_bytes(128, bits)
    guard = torch.full((w.num_blocks + 1, 16, 2, RB), 7, dtype=torch.uint8, device="cuda")
    pages = guard[:w.num_blocks]
    slots = torch.from_numpy(w.slots).cuda().clone()
    slots[5] = w.num_blocks * 16
    slots[9] = w.num_blocks * 16 + 3
    print(f"[qjl] out-of-range slots 5 and 9 of {w.num_tokens}", flush=True)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.write_kv_prod(ctx, torch.from_numpy(w.rows("k")).cuda(), pages, slots, bits, S, err_count=err,
                      check_slots=False)
    torch.cuda.synchronize()
    assert int(err.item()) == 2
    assert bool((guard[w.num_blocks] == 7).all())
    with pytest.raises(api.TQError):
        api.write_kv_prod(ctx, torch.from_numpy(w.rows("k")).cuda(), pages, slots, bits, S)


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_scores_half_precision_queries(ctx, dt):
    # fp16 / bf16 queries: the oracle scores the same rounded values
    bits = 3
    w = workloads.make_workload("qjlq", num_q_heads=8, num_kv_heads=2, seq_lens=[200, 37], seed=133)
    S = workloads.qjl_matrix(128, seed=11)
    signs = oracle.rht_signs(42, 128)
    shape = (w.num_blocks, 16, 2, oracle.prod_row_bytes(128, bits))
    pages, _, _ = oracle.write_prod(w.rows("k"), np.zeros(shape, np.uint8), w.slots, bits, signs, S)
    tq = torch.from_numpy(w.queries()).to(dt)
    q = tq.float().numpy()
    print(f"[qjl] scores with {dt} queries", flush=True)
    ref = oracle.paged_prod_scores(q, pages, w.block_table, w.seq_lens, bits, signs, S)
    got = api.prod_scores(ctx, tq.cuda(), torch.from_numpy(pages).cuda(), torch.from_numpy(w.block_table).cuda(),
                          torch.from_numpy(w.seq_lens).cuda(), bits, torch.from_numpy(S).cuda()).cpu().numpy()
    norms = np.zeros(ref.shape)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        t = np.arange(L)
        n = oracle.prod_bytes_to_rows(pages[w.block_table[b, t // 16], t % 16], bits, 128)[1].astype(np.float64)
        norms[b, :, :L] = np.repeat(n.T, 4, axis=0)
    _check_scores(got, ref, q, norms, f"scores {dt}")


@pytest.mark.parametrize("bits", [2, 4])
def test_writer_bf16_rows(ctx, bits):
    # bf16 raw rows (exact in fp32, which the oracle encodes), slots reversed
    t = torch.randn(40, 2, 128, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    raw32 = t.float().numpy()
    slots = np.arange(40, dtype=np.int64)[::-1].copy()
    S = workloads.qjl_matrix(128, seed=12 + bits)
    signs = oracle.rht_signs(42, 128)
    shape = (3, 16, 2, oracle.prod_row_bytes(128, bits))
    print(f"[qjl] writer bits={bits} bf16 rows", flush=True)
    ref, near_i, near_s = oracle.write_prod(raw32, np.zeros(shape, np.uint8), slots, bits, signs, S)
    pg = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    api.write_kv_prod(ctx, t.cuda(), pg, torch.from_numpy(slots).cuda(), bits, torch.from_numpy(S).cuda())
    torch.cuda.synchronize()
    got = pg.cpu().numpy()
    _compare_rows(got[slots // 16, slots % 16], ref[slots // 16, slots % 16], near_i[slots // 16, slots % 16],
                  near_s[slots // 16, slots % 16], bits, f"bf16 bits {bits}")


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_writer_special_rows(ctx, bits, dt):
    # a zero row (its residual is the constant cpos[0]), a one-hot row, constant
    # rows, a row with an exact fp32 norm tie, and extreme magnitudes (fp32
    # 1e-20 and 1e18, fp16 subnormals and 1e4): the MSE writer's special rows
    d = 128
    rng = np.random.default_rng(1)
    x = np.zeros((8, 1, d), np.float64)
    x[1, 0, [0, 1, 2, 3]] = [1.0, 2.0**-12, 2.0**-12, 2.0**-24]
    x[2, 0, 77] = -3.0
    x[3, 0] = 1.0
    x[4, 0, ::2] = 0.5
    x[5, 0] = rng.standard_normal(d)
    if dt == np.float32:
        x[6, 0] = rng.standard_normal(d) * 1e-20
        x[7, 0] = rng.standard_normal(d) * 1e18
    else:
        x[6, 0] = rng.integers(1, 30, d) * 2.0**-24
        x[7, 0] = rng.standard_normal(d) * 1e4
    x = x.astype(dt)
    S = workloads.qjl_matrix(128, seed=13)
    signs = oracle.rht_signs(42, 128)
    shape = (1, 8, 1, oracle.prod_row_bytes(128, bits))
    slots = np.arange(8, dtype=np.int64)
    print(f"[qjl] writer special rows bits={bits} {np.dtype(dt).name}", flush=True)
    ref, near_i, near_s = oracle.write_prod(x, np.zeros(shape, np.uint8), slots, bits, signs, S)
    pg = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    api.write_kv_prod(ctx, torch.from_numpy(x).cuda(), pg, torch.from_numpy(slots).cuda(), bits,
                      torch.from_numpy(S).cuda())
    torch.cuda.synchronize()
    _compare_rows(pg.cpu().numpy()[0], ref[0], near_i[0], near_s[0], bits, f"special rows bits {bits}",
                  check_fraction=False)
