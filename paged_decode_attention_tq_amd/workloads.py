"""Seeded synthetic inputs for the packed-page KV path.

This module only draws random numbers and lays them out (lengths, block
tables, slot maps, raw K/V rows, queries).  It contains none of the codec or
attention arithmetic, so both the HIP path and the CPU oracle can consume its
output.

Every random stream is a ``numpy.random.PCG64`` seeded from
``SeedSequence(seed, spawn_key=key)``:

* key ``(0,)``  -- layout: sequence lengths, the block-table permutation, the
  outlier channels and the dropped slots, drawn in that order;
* key ``(1, b)`` / ``(2, b)`` -- the raw K / V rows of sequence ``b``
  (``float32`` normals, then the optional per-token LogNormal scales);
* key ``(3,)`` -- the queries.

Per-sequence streams let a test regenerate just the sequences it samples.
Values are drawn in float32 and rounded once to the stored dtype.
"""

from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["Workload", "make_workload", "PRESETS", "preset", "random_pages", "qjl_matrix"]


def _rng(seed, *key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


@dataclasses.dataclass
class Workload:
    name: str
    head_dim: int
    k_bits: int
    v_bits: int
    num_q_heads: int
    num_kv_heads: int
    block_size: int
    seq_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, max_blocks_per_seq]
    num_blocks: int
    slots: np.ndarray  # int64 [N] (tokens of all sequences, in (b, t) order)
    dtype: type  # np.float16 or np.float32
    seed: int
    rht_seed: int = 42
    lognormal_sigma: float | None = None  # per-token norm scale of K and V
    outliers: np.ndarray | None = None  # int [n, 2] (kv_head, channel) pairs scaled x8
    outlier_scale: float = 8.0

    # ---- sizes -------------------------------------------------------------
    @property
    def batch(self):
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self):
        return int(self.seq_lens.sum())

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if self.batch else 0

    @property
    def cu_seqlens(self):
        return np.concatenate([[0], np.cumsum(self.seq_lens, dtype=np.int64)])

    def row_bytes(self, bits):
        return (self.head_dim * bits + 7) // 8 + 4

    def page_shape(self, bits):
        return (self.num_blocks, self.block_size, self.num_kv_heads, self.row_bytes(bits))

    def packed_kv_bytes(self):
        """Sum over sequences of L_b * Hkv * (RB_k + RB_v)."""
        return self.num_tokens * self.num_kv_heads * (self.row_bytes(self.k_bits) + self.row_bytes(self.v_bits))

    # ---- raw rows ----------------------------------------------------------
    def seq_rows(self, component: str, b: int) -> np.ndarray:
        """Raw rows ``[L_b, Hkv, d]`` of sequence ``b`` for component 'k' or 'v'."""
        key = {"k": 1, "v": 2}[component]
        L = int(self.seq_lens[b])
        rng = _rng(self.seed, key, b)
        x = rng.standard_normal((L, self.num_kv_heads, self.head_dim), dtype=np.float32)
        if self.lognormal_sigma is not None:
            s = rng.lognormal(0.0, self.lognormal_sigma, size=L).astype(np.float32)
            x *= s[:, None, None]
        if self.outliers is not None and len(self.outliers):
            x[:, self.outliers[:, 0], self.outliers[:, 1]] *= np.float32(self.outlier_scale)
        return x.astype(self.dtype)

    def rows(self, component: str, threads: int = 8) -> np.ndarray:
        """All raw rows ``[N, Hkv, d]`` in (b, t) order (matches ``slots``)."""
        out = np.empty((self.num_tokens, self.num_kv_heads, self.head_dim), dtype=self.dtype)
        cu = self.cu_seqlens

        def fill(b):
            out[cu[b] : cu[b + 1]] = self.seq_rows(component, b)

        with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            list(ex.map(fill, range(self.batch)))
        return out

    def queries(self) -> np.ndarray:
        """Queries ``[B, Hq, d]``."""
        rng = _rng(self.seed, 3)
        q = rng.standard_normal((self.batch, self.num_q_heads, self.head_dim), dtype=np.float32)
        if self.outliers is not None and len(self.outliers):
            G = self.num_q_heads // self.num_kv_heads
            for g, ch in self.outliers:
                q[:, g * G : (g + 1) * G, ch] *= np.float32(self.outlier_scale)
        return q.astype(self.dtype)

    def zero_pages(self, bits) -> np.ndarray:
        return np.zeros(self.page_shape(bits), dtype=np.uint8)

    def recent_window(self, cap: int, recent_lens, seed: int = 0):
        """Dense recent-window rows ``(k, v)``, each ``[B, cap, Hkv, d]`` in the
        workload's dtype, drawn like its K/V rows (N(0,1), the per-token
        LogNormal scale, the outlier channels) from the streams ``(5, b)`` /
        ``(6, b)`` of ``seed``; rows past ``recent_lens[b]`` are drawn too (a
        reader must ignore them)."""
        lens = np.asarray(recent_lens)
        if lens.shape != (self.batch,) or np.any(lens < 0) or np.any(lens > cap):
            raise ValueError("recent_lens must be [B] in 0..cap")
        out = []
        for key in (5, 6):
            x = np.empty((self.batch, cap, self.num_kv_heads, self.head_dim), dtype=np.float32)
            for b in range(self.batch):
                rng = _rng(seed, key, b)
                x[b] = rng.standard_normal((cap, self.num_kv_heads, self.head_dim), dtype=np.float32)
                if self.lognormal_sigma is not None:
                    x[b] *= rng.lognormal(0.0, self.lognormal_sigma, size=cap).astype(np.float32)[:, None, None]
            if self.outliers is not None and len(self.outliers):
                x[:, :, self.outliers[:, 0], self.outliers[:, 1]] *= np.float32(self.outlier_scale)
            out.append(x.astype(self.dtype))
        return out[0], out[1]


def make_workload(
    name,
    *,
    head_dim=128,
    k_bits=4,
    v_bits=4,
    num_q_heads,
    num_kv_heads,
    block_size=16,
    seq_lens=None,
    batch=None,
    seq_len=None,
    len_range=None,
    permute_pages=True,
    extra_blocks=0,
    dtype=np.float16,
    seed=42,
    rht_seed=42,
    lognormal_sigma=None,
    outlier_frac=None,
    drop_frac=None,
):
    """Build a workload.

    Lengths: ``seq_lens`` (explicit), or ``batch`` x ``seq_len``, or ``batch``
    lengths uniform on ``len_range = (lo, hi)`` inclusive.  Pages: each
    sequence owns ceil(L_b / block_size) pages; with ``permute_pages`` the
    physical page ids are a seeded permutation of all pages (assigned in
    sequence order), otherwise the identity.  ``extra_blocks`` unused pages
    are appended.  ``outlier_frac``: exactly round(frac * Hkv * d) distinct
    (kv_head, channel) pairs are scaled by 8 in K, V and the matching query
    heads.  ``drop_frac``: exactly round(frac * N) distinct tokens get slot -1.
    """
    g = _rng(seed, 0)
    if seq_lens is None:
        if len_range is not None:
            lo, hi = len_range
            seq_lens = g.integers(lo, hi, endpoint=True, size=batch)
        else:
            seq_lens = np.full(batch, seq_len)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = seq_lens.shape[0]
    npages = (seq_lens.astype(np.int64) + block_size - 1) // block_size
    total_pages = int(npages.sum())
    num_blocks = total_pages + int(extra_blocks)
    ids = g.permutation(total_pages) if permute_pages else np.arange(total_pages)
    max_pages = max(1, int(npages.max()) if B else 1)
    block_table = np.zeros((B, max_pages), dtype=np.int32)
    start = 0
    for b in range(B):
        block_table[b, : npages[b]] = ids[start : start + npages[b]]
        start += npages[b]
    outliers = None
    if outlier_frac:
        n_out = int(round(outlier_frac * num_kv_heads * head_dim))
        flat = g.choice(num_kv_heads * head_dim, size=n_out, replace=False)
        outliers = np.stack([flat // head_dim, flat % head_dim], axis=1)
    # flat slots of every token, (b, t) order
    N = int(seq_lens.sum())
    slots = np.empty(N, dtype=np.int64)
    pos = 0
    for b in range(B):
        L = int(seq_lens[b])
        t = np.arange(L, dtype=np.int64)
        slots[pos : pos + L] = block_table[b, t // block_size].astype(np.int64) * block_size + t % block_size
        pos += L
    if drop_frac:
        n_drop = int(round(drop_frac * N))
        slots[g.choice(N, size=n_drop, replace=False)] = -1
    return Workload(
        name=name,
        head_dim=head_dim,
        k_bits=k_bits,
        v_bits=v_bits,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        block_size=block_size,
        seq_lens=seq_lens,
        block_table=block_table,
        num_blocks=num_blocks,
        slots=slots,
        dtype=dtype,
        seed=seed,
        rht_seed=rht_seed,
        lognormal_sigma=lognormal_sigma,
        outliers=outliers,
    )


#: The five named workloads (tiny, the pages' geometry, mixed bits,
#: long context, ragged write + decode).
PRESETS = {
    "tiny": dict(k_bits=4, v_bits=4, num_q_heads=2, num_kv_heads=1, batch=1, seq_len=64,
                 permute_pages=False, dtype=np.float32, seed=42),
    "pages_geometry": dict(k_bits=4, v_bits=4, num_q_heads=16, num_kv_heads=2, batch=32,
                           seq_len=2048, lognormal_sigma=0.5, seed=42),
    "mixed_bits": dict(k_bits=4, v_bits=2, num_q_heads=32, num_kv_heads=8, batch=64,
                       seq_len=8192, outlier_frac=0.01, seed=42),
    "long_context": dict(k_bits=4, v_bits=4, num_q_heads=64, num_kv_heads=8, batch=8,
                         seq_len=131072, seed=42),
    "ragged_write": dict(k_bits=3, v_bits=3, num_q_heads=32, num_kv_heads=4, batch=256,
                         len_range=(1, 32768), drop_frac=0.10, seed=7),
}


def preset(name: str, **overrides) -> Workload:
    kw = dict(PRESETS[name])
    kw.update(overrides)
    return make_workload(name, **kw)


def random_pages(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, bits: int,
                 seed: int = 0) -> np.ndarray:
    """Page bytes ``uint8 [NB, BS, Hkv, RB]`` whose rows hold uniform random
    index bytes and a random positive float32 norm (last four bytes,
    little-endian), from the stream ``(4,)`` of ``seed``.  No row is encoded:
    these are inputs for readers of pages, not outputs of a writer."""
    ib = (head_dim * bits + 7) // 8
    g = _rng(seed, 4)
    shape = (num_blocks, block_size, num_kv_heads)
    idx = g.integers(0, 256, size=shape + (ib,), dtype=np.uint8)
    norm = (math.sqrt(head_dim) * g.lognormal(0.0, 0.5, size=shape)).astype("<f4")
    return np.concatenate([idx, norm[..., None].view(np.uint8)], axis=-1)


def qjl_matrix(d: int = 128, seed: int = 0) -> np.ndarray:
    """A ``d x d`` float32 matrix of i.i.d. N(0, 1) entries (stream ``(7,)`` of
    ``seed``): the sketch matrix of the prod key codec, an input of both the
    GPU path and the oracle."""
    return _rng(seed, 7).standard_normal((d, d), dtype=np.float32)

